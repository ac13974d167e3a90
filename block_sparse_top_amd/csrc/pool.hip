// Step 1 of block selection: per-block mean of q and k (or, as an option, the elementwise
// maximum over the block's tokens: the "in-block extremum" scoring that the MSA page's §2.2
// table lists for block-based methods).
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"), section
// "SparseFormer 注意力实现", step 1: q and k [B, N, H, D] are viewed as
// [B, num_blocks, block_size, H, D] and averaged over the block_size axis. The pooled blocks
// are stored [B, H, nb, D] in fp32 so that each (batch, head) row set is contiguous for the
// score step.
//
// Overlapping key blocks (the MSA page's §5.3 overlap remedy): key block j pools the tokens
// [j*stride, min(j*stride + block, N)); a shorter last block is averaged over its own tokens.
//
// The kernel is HBM-bound: every input byte is read once with 16-byte loads (overlapping key
// blocks read their shared tokens twice). One work-group reduces one (batch, block) of one
// tensor: the block is up to `block` consecutive token rows of H*D elements each, i.e. one
// contiguous span. Threads own 16-byte columns of a row and walk the tokens; partial sums of
// token groups meet in LDS.
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;                 // 16-byte loads in flight per thread

// Every input byte is read exactly once: stream it past the caches (nontemporal load).
__device__ __forceinline__ u32x4 load16(const uint8_t* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

struct PoolArgs {
  const uint8_t* x;   // [B, N, H, D] storage
  float* out;         // [B, H, nblk, D]
  int H;
  int64_t nblk;       // blocks of this tensor
  int stride;         // tokens between block starts (block, or the key stride)
};

// fold one 16-byte vector into the accumulators: sum, or elementwise max when pmax
template <int KIND>
__device__ __forceinline__ void fold(bool pmax, const u32x4& w, float* acc) {
  if (pmax) Vec<KIND>::vmax(w, acc); else Vec<KIND>::add(w, acc);
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void pool_kernel(PoolArgs qa, PoolArgs ka, int64_t nmax,
                                                        int64_t N, int D, int block,
                                                        float inv_block, bool pmax) {
  constexpr int E = Vec<KIND>::E;
  // loads in flight per thread: an fp8 vector widens to 16 floats and the compiler converts
  // all loads of a batch before adding them, so fp8 takes 4 at a time (121 registers, four
  // waves per SIMD; 16 at a time cost 272 registers, one wave per SIMD)
  constexpr int U = KIND == 2 ? 4 : kUnroll;
  const float init = pmax ? -__builtin_inff() : 0.f;
  extern __shared__ float red[];                       // [T][V*E] partial sums
  const PoolArgs a = blockIdx.y == 0 ? qa : ka;
  const int64_t bi = blockIdx.x;                       // b * nmax + i
  const int64_t b = bi / nmax, i = bi - b * nmax;
  if (i >= a.nblk) return;                             // the other tensor has more blocks
  const int64_t first = i * a.stride;                  // first token of block (b, i)
  const int cnt = N - first < block ? (int)(N - first) : block;   // its tokens
  const int V = a.H * D / E;                           // 16-byte vectors per token row
  const int64_t row_bytes = (int64_t)V * 16;
  const uint8_t* base = a.x + (b * N + first) * row_bytes;
  const float scale = pmax ? 1.0f : cnt == block ? inv_block : 1.0f / (float)cnt;
  const int tid = threadIdx.x;
  const int nblk = (int)a.nblk;

  if (V <= kThreads) {
    const int T = kThreads / V;                        // token groups
    const int c = tid % V, grp = tid / V;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = init;
    if (grp < T) {
      const uint8_t* p = base + (int64_t)c * 16;
      int t = grp;
      for (; t + (U - 1) * T < cnt; t += U * T) {     // U loads in flight
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = load16(p + (int64_t)(t + u * T) * row_bytes);
        if (pmax) {
#pragma unroll
          for (int u = 0; u < U; ++u) Vec<KIND>::vmax(w[u], acc);
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u) Vec<KIND>::add(w[u], acc);
        }
      }
      for (; t < cnt; t += T) fold<KIND>(pmax, load16(p + (int64_t)t * row_bytes), acc);
#pragma unroll
      for (int e = 0; e < E; ++e) red[grp * V * E + c * E + e] = acc[e];
    }
    __syncthreads();
    for (int o = tid; o < V * E; o += kThreads) {
      float s = init;
      for (int g2 = 0; g2 < T; ++g2)
        s = pmax ? fmaxf(s, red[g2 * V * E + o]) : s + red[g2 * V * E + o];
      const int h = o / D, d = o - h * D;
      a.out[(((int64_t)b * a.H + h) * nblk + i) * D + d] = s * scale;
    }
  } else {
    for (int c = tid; c < V; c += kThreads) {
      float acc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = init;
      const uint8_t* p = base + (int64_t)c * 16;
      int t = 0;
      for (; t + U - 1 < cnt; t += U) {
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = load16(p + (int64_t)(t + u) * row_bytes);
        if (pmax) {
#pragma unroll
          for (int u = 0; u < U; ++u) Vec<KIND>::vmax(w[u], acc);
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u) Vec<KIND>::add(w[u], acc);
        }
      }
      for (; t < cnt; ++t) fold<KIND>(pmax, load16(p + (int64_t)t * row_bytes), acc);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int o = c * E + e;
        const int h = o / D, d = o - h * D;
        a.out[(((int64_t)b * a.H + h) * nblk + i) * D + d] = acc[e] * scale;
      }
    }
  }
}

}  // namespace

hipError_t launch_pool(int kind, int which, int64_t B, int64_t N, int Hq, int Hkv, int D,
                       int block, int key_stride, int64_t nkb, const void* q, const void* k,
                       float* qbar, float* kbar, bool pmax, hipStream_t stream) {
  const int64_t nb = N / block;
  const int ebytes = kind == 0 ? 4 : kind == 1 ? 2 : 1;
  const int E = 16 / ebytes;
  // LDS for the partial sums: T * V * E floats with T = 256 / V, i.e. at most 256 * E.
  size_t lds = 0;
  for (int H : {which & 1 ? Hq : Hkv, which & 2 ? Hkv : Hq}) {
    int V = H * D / E;
    if (V <= kThreads) {
      size_t s = (size_t)(kThreads / V) * V * E * sizeof(float);
      lds = s > lds ? s : lds;
    }
  }
  PoolArgs qa{(const uint8_t*)q, qbar, Hq, nb, block};
  PoolArgs ka{(const uint8_t*)k, kbar, Hkv, nkb, key_stride};
  if (which == 2) qa = ka;                             // k only: grid.y == 1 reads qa
  const int64_t nmax = which == 1 ? nb : which == 2 ? nkb : (nb > nkb ? nb : nkb);
  dim3 grid((unsigned)(B * nmax), which == 3 ? 2 : 1);
  const float inv = 1.0f / (float)block;               // exact for power-of-two blocks
  switch (kind) {
    case 0: pool_kernel<0><<<grid, kThreads, lds, stream>>>(qa, ka, nmax, N, D, block, inv, pmax); break;
    case 1: pool_kernel<1><<<grid, kThreads, lds, stream>>>(qa, ka, nmax, N, D, block, inv, pmax); break;
    default: pool_kernel<2><<<grid, kThreads, lds, stream>>>(qa, ka, nmax, N, D, block, inv, pmax); break;
  }
  return hipGetLastError();
}

}  // namespace bsattn
