// Step 1 of block selection: per-block mean of q and k.
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"), section
// "SparseFormer 注意力实现", step 1: q and k [B, N, H, D] are viewed as
// [B, num_blocks, block_size, H, D] and averaged over the block_size axis. The pooled blocks
// are stored [B, H, nb, D] in fp32 so that each (batch, head) row set is contiguous for the
// score step.
//
// The kernel is HBM-bound: every input byte is read once with 16-byte loads. One work-group
// reduces one (batch, block) of one tensor: the block is `block` consecutive token rows of
// H*D elements each, i.e. one contiguous span of block*H*D elements. Threads own 16-byte
// columns of a row and walk the tokens; partial sums of token groups meet in LDS.
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

constexpr int kThreads = 256;

// Elements per 16-byte vector and their fp32 values, per storage kind.
template <int KIND> struct Vec;
template <> struct Vec<0> {            // fp32
  static constexpr int E = 4;
  __device__ static void add(const u32x4& w, float* a) {
    a[0] += __uint_as_float(w.x); a[1] += __uint_as_float(w.y);
    a[2] += __uint_as_float(w.z); a[3] += __uint_as_float(w.w);
  }
};
template <> struct Vec<1> {            // bf16
  static constexpr int E = 8;
  __device__ static void add(const u32x4& w, float* a) {
    a[0] += bf16lo(w.x); a[1] += bf16hi(w.x); a[2] += bf16lo(w.y); a[3] += bf16hi(w.y);
    a[4] += bf16lo(w.z); a[5] += bf16hi(w.z); a[6] += bf16lo(w.w); a[7] += bf16hi(w.w);
  }
};
template <> struct Vec<2> {            // OCP fp8 e4m3 (gfx950 converts the OCP format)
  static constexpr int E = 16;
  __device__ static void add(const u32x4& w, float* a) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], false);
      auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[i], true);
      a[4 * i + 0] += lo[0]; a[4 * i + 1] += lo[1];
      a[4 * i + 2] += hi[0]; a[4 * i + 3] += hi[1];
    }
  }
};

struct PoolArgs {
  const uint8_t* x;   // [B, N, H, D] storage
  float* out;         // [B, H, nb, D]
  int H;
};

template <int KIND>
__global__ __launch_bounds__(kThreads) void pool_kernel(PoolArgs qa, PoolArgs ka, int64_t nb,
                                                        int D, int block, float inv_block) {
  constexpr int E = Vec<KIND>::E;
  extern __shared__ float red[];                       // [T][V*E] partial sums
  const PoolArgs a = blockIdx.y == 0 ? qa : ka;
  const int64_t bi = blockIdx.x;                       // b * nb + i
  const int64_t b = bi / nb, i = bi - b * nb;
  const int V = a.H * D / E;                           // 16-byte vectors per token row
  const int64_t row_bytes = (int64_t)V * 16;
  const uint8_t* base = a.x + bi * block * row_bytes;  // first token of block (b, i)
  const int tid = threadIdx.x;

  if (V <= kThreads) {
    const int T = kThreads / V;                        // token groups
    const int c = tid % V, grp = tid / V;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    if (grp < T) {
      const uint8_t* p = base + (int64_t)c * 16;
      int t = grp;
      for (; t + 7 * T < block; t += 8 * T) {          // 8 loads in flight
        u32x4 w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          w[u] = *(const u32x4*)(p + (int64_t)(t + u * T) * row_bytes);
#pragma unroll
        for (int u = 0; u < 8; ++u) Vec<KIND>::add(w[u], acc);
      }
      for (; t < block; t += T) Vec<KIND>::add(*(const u32x4*)(p + (int64_t)t * row_bytes), acc);
#pragma unroll
      for (int e = 0; e < E; ++e) red[grp * V * E + c * E + e] = acc[e];
    }
    __syncthreads();
    for (int o = tid; o < V * E; o += kThreads) {
      float s = 0.f;
      for (int g2 = 0; g2 < T; ++g2) s += red[g2 * V * E + o];
      const int h = o / D, d = o - h * D;
      a.out[(((int64_t)b * a.H + h) * nb + i) * D + d] = s * inv_block;
    }
  } else {
    for (int c = tid; c < V; c += kThreads) {
      float acc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = 0.f;
      const uint8_t* p = base + (int64_t)c * 16;
      int t = 0;
      for (; t + 7 < block; t += 8) {
        u32x4 w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) w[u] = *(const u32x4*)(p + (int64_t)(t + u) * row_bytes);
#pragma unroll
        for (int u = 0; u < 8; ++u) Vec<KIND>::add(w[u], acc);
      }
      for (; t < block; ++t) Vec<KIND>::add(*(const u32x4*)(p + (int64_t)t * row_bytes), acc);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int o = c * E + e;
        const int h = o / D, d = o - h * D;
        a.out[(((int64_t)b * a.H + h) * nb + i) * D + d] = acc[e] * inv_block;
      }
    }
  }
}

}  // namespace

hipError_t launch_pool(int kind, int64_t B, int64_t N, int Hq, int Hkv, int D, int block,
                       const void* q, const void* k, float* qbar, float* kbar,
                       hipStream_t stream) {
  const int64_t nb = N / block;
  const int ebytes = kind == 0 ? 4 : kind == 1 ? 2 : 1;
  const int E = 16 / ebytes;
  // LDS for the partial sums: T * V * E floats with T = 256 / V, i.e. at most 256 * E.
  size_t lds = 0;
  for (int H : {Hq, Hkv}) {
    int V = H * D / E;
    if (V <= kThreads) {
      size_t s = (size_t)(kThreads / V) * V * E * sizeof(float);
      lds = s > lds ? s : lds;
    }
  }
  PoolArgs qa{(const uint8_t*)q, qbar, Hq};
  PoolArgs ka{(const uint8_t*)k, kbar, Hkv};
  dim3 grid((unsigned)(B * nb), 2);
  const float inv = 1.0f / (float)block;               // exact for power-of-two blocks
  switch (kind) {
    case 0: pool_kernel<0><<<grid, kThreads, lds, stream>>>(qa, ka, nb, D, block, inv); break;
    case 1: pool_kernel<1><<<grid, kThreads, lds, stream>>>(qa, ka, nb, D, block, inv); break;
    default: pool_kernel<2><<<grid, kThreads, lds, stream>>>(qa, ka, nb, D, block, inv); break;
  }
  return hipGetLastError();
}

}  // namespace bsattn
