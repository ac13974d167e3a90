// Steps 2-3 of block selection for many key blocks (nb > 1024): the score matrix is built in
// the workspace by an fp32 MFMA product, then each row's top-k is found by one work-group.
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"), section
// "SparseFormer 注意力实现": block_scores = einsum over d of the pooled query and key blocks
// (no scale), then torch.topk with k = int(topk_ratio * num_blocks) per row. MSA page
// ("从M2.7到M3：多模态模型稀疏注意力架构设计与实现全解析") §3.2: 1M-token context at block 128, i.e.
// 8192 key blocks per row; §3.3: block scores as a matrix product.
//
// score_gemm_kernel: S[b,h] = qbar[b,h] (nb x D) * kbar[b,g]^T, fp32, unscaled. One wave
// computes a 64x64 tile with v_mfma_f32_32x32x2_f32 (four 32x32 sub-tiles); the lane half h of
// k-step s carries d = s + (D/2)*h on both operands, so every lane reads contiguous halves of
// its query and key rows. Every score goes through the same instruction sequence, so equal
// pooled key blocks give bit-equal scores.
//
// topk_rows_kernel: one work-group (256 threads) per row; thread t holds the 32-column chunk
// j = 32t .. 32t+31 (nb = 8192) as order-preserving keys. A threshold T is built bit by bit
// (block-wide counts of keys >= candidate; early exit once exactly k keys are >= T), keys > T
// are kept and keys == T fill the remaining places in ascending j (the lower index wins).
// Output positions come from block-wide exclusive scans, so the row is written in ascending j.
// Causal option: as in the fused kernel, columns j > i get key 0, column i the largest key,
// the row keeps min(topk, i+1) blocks and its remaining places are set to -1.
//
// Group-shared selection (GQA, MSA §3.1): group_sum_kernel adds the pooled queries of each
// group's G heads into the rows of its first head (the scores of the sum are the sum of the
// heads' scores), the product runs once per (batch, KV head) on those rows, and each row's
// top-k is written to the idx rows of all G heads.
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

typedef float f32x16v __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- score GEMM
__global__ __launch_bounds__(64) void score_gemm_kernel(const float* __restrict__ qbar,
                                                        const float* __restrict__ kbar,
                                                        float* __restrict__ S, int Hq, int Hkv,
                                                        int nb, int D, int tiles, bool group) {
  // tile index: (b*HS + s) * tiles^2 + ti * tiles + tj, 64x64 each, s a selection head (a
  // query head, or a KV head whose group's summed queries sit in the rows of its first head);
  // tiles of one (batch, selection head) share their pooled rows: keep them on one XCD's L2
  const int G = Hq / Hkv, HS = group ? Hkv : Hq;
  const int64_t t = xcd_remap(blockIdx.x, gridDim.x);
  const int tj = (int)(t % tiles), ti = (int)((t / tiles) % tiles);
  const int64_t bh = t / ((int64_t)tiles * tiles);   // b * HS + s
  const int sh = (int)(bh % HS), b = (int)(bh / HS);
  const int hq = group ? sh * G : sh;                 // query head of the pooled rows
  const int g = group ? sh : sh / G;
  const float* Q = qbar + ((int64_t)b * Hq + hq) * nb * D;
  const float* K = kbar + ((int64_t)b * Hkv + g) * nb * D;
  const int lane = threadIdx.x, l32 = lane & 31, half = lane >> 5;
  const int half_d = D / 2;

  f32x16v acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;

  const float* qrow[2];
  const float* krow[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    qrow[a] = Q + (int64_t)(ti * 64 + 32 * a + l32) * D + half * half_d;
    krow[a] = K + (int64_t)(tj * 64 + 32 * a + l32) * D + half * half_d;
  }
  // the operands of step s0 + 4 are loaded while step s0 multiplies
  f32x4 qa[2], kb[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    qa[a] = *(const f32x4*)(qrow[a]);
    kb[a] = *(const f32x4*)(krow[a]);
  }
  for (int s0 = 0; s0 < half_d; s0 += 4) {
    f32x4 qn[2], kn[2];
    const int sn = s0 + 4 < half_d ? s0 + 4 : s0;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      qn[a] = *(const f32x4*)(qrow[a] + sn);
      kn[a] = *(const f32x4*)(krow[a] + sn);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[a][e], kb[c][e], acc[a][c], 0, 0, 0);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      qa[a] = qn[a];
      kb[a] = kn[a];
    }
  }
  // acc[a][c][r]: row ti*64 + 32a + 8(r/4) + 4*half + r%4, column tj*64 + 32c + l32
  float* Sbh = S + bh * nb * nb;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = ti * 64 + 32 * a + 8 * (r >> 2) + 4 * half + (r & 3);
        Sbh[(int64_t)row * nb + tj * 64 + 32 * c + l32] = acc[a][c][r];
      }
}

// ---------------------------------------------------------------- per-row top-k
constexpr int kTopkThreads = 256;
constexpr int kPerThread = 32;             // columns per thread: nb <= 8192

__device__ __forceinline__ int block_sum(int v, int* red) {
  // wave sum (DPP within 16 lanes, then across 16 and 32 lanes), then the 4 wave sums
  // through LDS (caller syncs around reuse)
  v = group_sum<16>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const int total = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return total;
}

// exclusive prefix of v over threads in thread order, and the block total
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) red[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < w) before += red[i];
    tot += red[i];
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

// rows of S: (b * HS + s) * nb + i; the top-k of a row goes to the idx rows of the G query
// heads s*G .. s*G+G-1 of a group (group), or of query head s
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(const float* __restrict__ S,
                                                                 int32_t* __restrict__ idx,
                                                                 int nb, int topk, bool causal,
                                                                 int G) {
  __shared__ int red[4];
  const int64_t row = blockIdx.x;
  const int i = (int)(row % nb);           // query block of this row
  const int lim = causal ? i + 1 : nb;     // admissible columns j < lim
  const int kr = causal && i + 1 < topk ? i + 1 : topk;
  const float* srow = S + row * nb;
  const int t = threadIdx.x;
  const int j0 = t * kPerThread;
  uint32_t key[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; e += 4) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (j0 + e < nb) v = *(const f32x4*)(srow + j0 + e);   // nb is a multiple of 4
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j0 + e + q;
      key[e + q] = j < lim ? (causal && j == i ? 0xFFFFFFFFu : order_key(v[q])) : 0u;
    }
  }
  // keys of columns past lim are 0: no candidate (>= 1) and no reached T (>= 1) counts them
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) c += key[e] >= cand;
    const int cnt = block_sum(c, red);
    if (cnt >= kr) T = cand;
    if (cnt == kr) break;
  }
  int gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    gt += key[e] > T;
    eq += (j0 + e < lim) && key[e] == T;
  }
  const int tot_gt = block_sum(gt, red);
  int tot_eq;
  const int eq_before = block_exclusive_scan(eq, red, &tot_eq);
  const int need = kr - tot_gt;            // places for keys equal to T
  int sel = 0;
  int eq_seen = eq_before;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const bool is_eq = (j0 + e < lim) && key[e] == T;
    sel += key[e] > T || (is_eq && eq_seen < need);
    eq_seen += is_eq;
  }
  int tot_sel;
  const int pos0 = block_exclusive_scan(sel, red, &tot_sel);
  const int64_t bs = row / nb;             // b * HS + s
  for (int hh = 0; hh < G; ++hh) {
    int32_t* out = idx + ((bs * G + hh) * nb + i) * topk;
    int pos = pos0;
    eq_seen = eq_before;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const bool is_eq = (j0 + e < lim) && key[e] == T;
      if (key[e] > T || (is_eq && eq_seen < need)) out[pos++] = j0 + e;
      eq_seen += is_eq;
    }
    for (int p = kr + t; p < topk; p += kTopkThreads) out[p] = -1;   // unused causal places
  }
}

// in place: rows of head g*G of each group += rows of heads g*G+1 .. g*G+G-1, in head order
__global__ __launch_bounds__(256) void group_sum_kernel(float* __restrict__ qbar, int64_t B,
                                                        int Hq, int Hkv, int64_t per_head) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (b, g, element)
  if (e >= B * Hkv * per_head) return;
  const int G = Hq / Hkv;
  const int64_t bg = e / per_head, x = e % per_head;
  float* first = qbar + bg * G * per_head + x;       // head g*G of batch b
  float s = first[0];
  for (int hh = 1; hh < G; ++hh) s += first[hh * per_head];
  first[0] = s;
}

}  // namespace

hipError_t launch_scores_large(int64_t B, int Hq, int Hkv, int nb, int D, float* qbar,
                               const float* kbar, float* S, bool group, hipStream_t stream) {
  if (group && Hq > Hkv) {
    const int64_t n = B * Hkv * (int64_t)nb * D;
    group_sum_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, stream>>>(
        qbar, B, Hq, Hkv, (int64_t)nb * D);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int tiles = nb / 64;
  const int64_t n = B * (group ? Hkv : Hq) * (int64_t)tiles * tiles;
  score_gemm_kernel<<<dim3((unsigned)n), 64, 0, stream>>>(qbar, kbar, S, Hq, Hkv, nb, D, tiles,
                                                          group);
  return hipGetLastError();
}

hipError_t launch_topk_rows(int64_t rows, int nb, int topk, const float* S, int32_t* idx,
                            bool causal, int G, hipStream_t stream) {
  topk_rows_kernel<<<dim3((unsigned)rows), kTopkThreads, 0, stream>>>(S, idx, nb, topk, causal,
                                                                      G);
  return hipGetLastError();
}

}  // namespace bsattn
