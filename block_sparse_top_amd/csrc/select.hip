// Steps 2-3 of block selection, fused: block scores and per-row top-k.
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"), section
// "SparseFormer 注意力实现": step 1 forms block_scores[b,h,i,j] = sum_d qbar[b,h,i,d] *
// kbar[b,h,j,d] (an einsum, no scale); step 2 keeps torch.topk(block_scores,
// k = int(topk_ratio * num_blocks)) per row. The MSA page ("从M2.7到M3：多模态模型稀疏注意力架构
// 设计与实现全解析", §3.3 计算优化) suggests computing the block scores as a matrix product and
// fusing kernels; here the score tile never leaves the chip.
//
// Layout: one work-group = 4 waves = 16 consecutive query-block rows of one (batch, query
// head). Key-block columns are staged through LDS 64 at a time, transposed to [D][64], so
// lane l owns columns j = l + 64*c. Scores are fp32, summed over d in order with fused
// multiply-adds, identically for every column (equal pooled key blocks give equal scores).
//
// Selection of one row is done by its wave with no sorting: scores map to order-preserving
// 32-bit keys, the k-th largest key T is built bit by bit from the top (a candidate bit stays
// when at least k keys are >= the candidate, counted with ballots), then every key > T is
// kept and the keys == T fill the remaining places in ascending j (the lower index wins a
// tie). Kept columns are compacted with ballot/mbcnt in ascending j order.
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 4;
constexpr int kRowsPerGroup = kRowsPerWave * (kThreads / kWave);  // 16

template <int CPL>  // score columns per lane: nb <= 64 * CPL
__global__ __launch_bounds__(kThreads) void score_select_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int32_t* __restrict__ idx,
    int Hq, int Hkv, int nb, int D, int topk, int row_tiles) {
  extern __shared__ float smem[];
  float* kT = smem;                         // [D][64] current column chunk, transposed
  float* qs = smem + D * 64;                // [16][D] query rows of this work-group

  const int tile = blockIdx.x;
  const int rt = tile % row_tiles;
  const int bh = tile / row_tiles;          // b * Hq + h
  const int h = bh % Hq, b = bh / Hq;
  const int g = h / (Hq / Hkv);
  const float* Q = qbar + (int64_t)bh * nb * D;
  const float* K = kbar + ((int64_t)b * Hkv + g) * nb * D;
  const int row0 = rt * kRowsPerGroup;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

  for (int e = tid; e < kRowsPerGroup * D; e += kThreads) {
    const int r = e / D;
    qs[e] = (row0 + r < nb) ? Q[(int64_t)(row0 + r) * D + (e - r * D)] : 0.f;
  }

  float acc[kRowsPerWave][CPL];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[r][c] = 0.f;

  const int D4 = D / 4;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    __syncthreads();                        // previous chunk consumed
    for (int e = tid; e < 64 * D4; e += kThreads) {
      const int col = e % 64, d4 = e / 64;
      const int j = c * 64 + col;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (j < nb) v = *(const f32x4*)(K + (int64_t)j * D + 4 * d4);
      kT[(4 * d4 + 0) * 64 + col] = v[0];
      kT[(4 * d4 + 1) * 64 + col] = v[1];
      kT[(4 * d4 + 2) * 64 + col] = v[2];
      kT[(4 * d4 + 3) * 64 + col] = v[3];
    }
    __syncthreads();
    const float* qw = qs + wave * kRowsPerWave * D;
    for (int d = 0; d < D; d += 4) {
      const float k0 = kT[(d + 0) * 64 + lane], k1 = kT[(d + 1) * 64 + lane];
      const float k2 = kT[(d + 2) * 64 + lane], k3 = kT[(d + 3) * 64 + lane];
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        const f32x4 qv = *(const f32x4*)(qw + r * D + d);
        float s = acc[r][c];
        s = __builtin_fmaf(qv[0], k0, s);
        s = __builtin_fmaf(qv[1], k1, s);
        s = __builtin_fmaf(qv[2], k2, s);
        s = __builtin_fmaf(qv[3], k3, s);
        acc[r][c] = s;
      }
    }
  }

  // ---- per-row top-k, one wave per row
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int row = row0 + wave * kRowsPerWave + r;
    if (row >= nb) break;                   // wave-uniform
    uint32_t key[CPL];
    bool valid[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      valid[c] = (c * 64 + lane) < nb;
      key[c] = valid[c] ? order_key(acc[r][c]) : 0u;
    }
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int c = 0; c < CPL; ++c) cnt += __popcll(__ballot(valid[c] && key[c] >= cand));
      if (cnt >= topk) T = cand;
    }
    int gt = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) gt += __popcll(__ballot(valid[c] && key[c] > T));
    const int need = topk - gt;             // >= 1 places for keys equal to T
    int32_t* out = idx + ((int64_t)bh * nb + row) * topk;
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const bool is_eq = valid[c] && key[c] == T;
      const uint64_t meq = __ballot(is_eq);
      const bool sel = valid[c] && (key[c] > T || (is_eq && eq_before + lanes_below(meq) < need));
      const uint64_t msel = __ballot(sel);
      if (sel) out[sel_before + lanes_below(msel)] = c * 64 + lane;
      eq_before += __popcll(meq);
      sel_before += __popcll(msel);
    }
  }
}

}  // namespace

hipError_t launch_score_select(int64_t B, int Hq, int Hkv, int64_t nb, int D, int topk,
                               const float* qbar, const float* kbar, int32_t* idx,
                               hipStream_t stream) {
  const int row_tiles = (int)((nb + kRowsPerGroup - 1) / kRowsPerGroup);
  const dim3 grid((unsigned)(B * Hq * row_tiles));
  const size_t lds = (size_t)(D * 64 + kRowsPerGroup * D) * sizeof(float);
  const int n = (int)nb;
  if (nb <= 64)
    score_select_kernel<1><<<grid, kThreads, lds, stream>>>(qbar, kbar, idx, Hq, Hkv, n, D, topk, row_tiles);
  else if (nb <= 128)
    score_select_kernel<2><<<grid, kThreads, lds, stream>>>(qbar, kbar, idx, Hq, Hkv, n, D, topk, row_tiles);
  else if (nb <= 256)
    score_select_kernel<4><<<grid, kThreads, lds, stream>>>(qbar, kbar, idx, Hq, Hkv, n, D, topk, row_tiles);
  else if (nb <= 512)
    score_select_kernel<8><<<grid, kThreads, lds, stream>>>(qbar, kbar, idx, Hq, Hkv, n, D, topk, row_tiles);
  else
    score_select_kernel<16><<<grid, kThreads, lds, stream>>>(qbar, kbar, idx, Hq, Hkv, n, D, topk, row_tiles);
  return hipGetLastError();
}

}  // namespace bsattn
