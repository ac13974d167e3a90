// Steps 1 (query side), 2 and 3 of block selection, fused: query-block pooling, block scores
// and per-row top-k. The key side is pooled beforehand (pool.hip), since every row needs all
// pooled key blocks.
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"), section
// "SparseFormer 注意力实现": step 1 forms block_scores[b,h,i,j] = sum_d qbar[b,h,i,d] *
// kbar[b,h,j,d] (an einsum, no scale); step 2 keeps torch.topk(block_scores,
// k = int(topk_ratio * num_blocks)) per row. The MSA page ("从M2.7到M3：多模态模型稀疏注意力架构
// 设计与实现全解析", §3.3 计算优化) suggests computing the block scores as a matrix product and
// fusing kernels; here the score rows never leave the chip.
//
// Layout: one work-group = 4 waves = 4*RW consecutive query-block rows of one (batch, query
// head). It first averages its rows' query tokens (16-byte loads, streamed past the caches:
// this phase is HBM-bound and overlaps the arithmetic of the other work-groups on the CU),
// keeps the pooled rows in LDS and also stores them to the workspace. Then each wave holds
// RW rows x CPL columns of scores in registers, lane l owning columns
// j = l + 64*c. Key-block columns are staged through LDS 64 at a time with coalesced row
// loads, kept row-major with a one-float pad (lane j reads row j: banks j + d, no conflict).
// Scores are fp32, summed over d in order with fused multiply-adds, identically for every
// column (equal pooled key blocks give equal scores).
//
// Selection of one row is done by its wave with no sorting: scores map to order-preserving
// 32-bit keys, and a threshold T is built bit by bit from the top (a candidate bit stays when
// at least k keys are >= the candidate, counted with ballots). The search stops as soon as
// exactly k keys are >= T (then T separates the top k); otherwise it runs to the last bit
// and T is the k-th largest key. Every key > T is kept and the keys == T fill the remaining
// places in ascending j (the lower index wins a tie). Kept columns are compacted with
// ballot/mbcnt in ascending j order.
//
// Options (flags): kPoolMax pools with the elementwise maximum instead of the mean.
// kCausal restricts row i to the key blocks j <= i and forces its own block: column j > i
// gets key 0 (never counted), column i the largest key, and the row keeps min(topk, i+1)
// blocks; its remaining places are set to -1. kGroup makes one selection per KV head: the
// work-group pools the rows of all G query heads of the group and sums them (the scores of
// the sum are the sum of the heads' scores), and the chosen blocks are written for each of
// the G heads; the pooled-query workspace rows of the group's first head hold the sums.
// nrand > 0 (random places): the row keeps its top topk - nrand blocks, then draw p takes the
// (x mod m_p)-th of the m_p = nk - (topk - nrand) - p blocks not yet chosen, in ascending
// order, x = element row * 2^16 + p of the SplitMix64 sequence (Steele, Lea, Flood, 2014)
// seeded with `seed`, row = (batch, selection head, query block) in C order.
// Rows are the nb query blocks, columns the nk key blocks: nk = nb, or more with overlapping
// key blocks (the MSA page's §5.3), whose pooled rows the key pool wrote (not with kCausal).
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// Small work-groups (8 rows) give ~5 rounds of work-groups per CU, so that the pooling loads
// of some overlap the score/select arithmetic of others. From 512 key blocks on, each
// work-group streams so many pooled keys through LDS that 16 rows share them (fp8 workload,
// 1024 key blocks: 1.88 -> 1.66 ms).
template <int CPL>
struct SelCfg {
  static constexpr int RW = CPL >= 8 ? 4 : 2;                   // rows per wave
  static constexpr int RG = kWaves * RW;                       // rows per work-group
};

template <int KIND, int CPL>  // storage kind; score columns per lane: nk <= 64 * CPL
__global__ __launch_bounds__(kThreads) void select_kernel(
    const uint8_t* __restrict__ q, float* __restrict__ qbar, const float* __restrict__ kbar,
    int32_t* __restrict__ idx, int64_t N, int Hq, int Hkv, int nb, int nk, int D, int block,
    int topk, int row_tiles, float inv_block, unsigned flags, int nrand, uint64_t seed) {
  constexpr int RW = SelCfg<CPL>::RW, RG = SelCfg<CPL>::RG;
  constexpr int E = Vec<KIND>::E;
  constexpr int EB = 16 / E;                // bytes per stored element
  extern __shared__ float smem[];
  const int KS = D + 1;                     // padded row stride of the key chunk
  float* ks = smem;                         // [64][D+1] current key-block chunk
  float* qs = smem + 64 * KS;               // [RG][D] pooled query rows of this work-group

  // work-groups of one (batch, head) read the same pooled keys: keep them on one XCD's L2
  const int tile = (int)xcd_remap(blockIdx.x, gridDim.x);
  const bool causal = flags & kCausal, pmax = flags & kPoolMax, group = flags & kGroup;
  const int G = Hq / Hkv;
  const int HS = group ? Hkv : Hq;          // selection heads
  const int rt = tile % row_tiles;
  const int sh = tile / row_tiles;          // b * HS + selection head
  const int b = sh / HS;
  const int g = group ? sh % HS : (sh % HS) / G;
  const int h0 = group ? g * G : sh % HS;   // first query head pooled here
  const int nh = group ? G : 1;             // query heads pooled and summed
  const int bh = b * Hq + h0;               // workspace row set of the pooled queries
  const float* K = kbar + ((int64_t)b * Hkv + g) * nk * D;
  const int row0 = rt * RG;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int D4 = D / 4;

  // ---- pool the RG query rows: pair (row r, 16-byte column c); TG token groups per pair
  const float init = pmax ? -__builtin_inff() : 0.f;
  const float scl = pmax ? 1.f : inv_block;
  for (int j = 0; j < nh; ++j) {
    const int h = h0 + j;
    const bool last = j == nh - 1;
    const int C16 = D / E;                  // 16-byte columns per token of one head
    const int pairs = RG * C16;
    const int per_pass = pairs < kThreads ? pairs : kThreads;
    const int TG = kThreads / per_pass;     // token groups (>= 1)
    const int64_t tok_bytes = (int64_t)Hq * D * EB;
    float* red = ks;                        // [TG][per_pass][E] partial sums (fits: D >= 64)
    for (int p0 = 0; p0 < pairs; p0 += per_pass) {
      const int pr = p0 + tid % per_pass, tg = tid / per_pass;
      const int r = pr / C16, c = pr % C16;
      const int row = row0 + r;
      float acc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = init;
      if (tg < TG && row < nb) {
        const uint8_t* src = q + (((int64_t)b * N + (int64_t)row * block) * Hq + h) * D * EB + c * 16;
        int t = tg;
        for (; t + 7 * TG < block; t += 8 * TG) {
          u32x4 w[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            w[u] = __builtin_nontemporal_load((const u32x4*)(src + (int64_t)(t + u * TG) * tok_bytes));
          if (pmax) {
#pragma unroll
            for (int u = 0; u < 8; ++u) Vec<KIND>::vmax(w[u], acc);
          } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) Vec<KIND>::add(w[u], acc);
          }
        }
        for (; t < block; t += TG) {
          const u32x4 w = __builtin_nontemporal_load((const u32x4*)(src + (int64_t)t * tok_bytes));
          if (pmax) Vec<KIND>::vmax(w, acc); else Vec<KIND>::add(w, acc);
        }
      }
      if (TG > 1) {
        __syncthreads();                    // previous pass done with red
        if (tg < TG)
#pragma unroll
          for (int e = 0; e < E; ++e) red[(tg * per_pass + tid % per_pass) * E + e] = acc[e];
        __syncthreads();
        for (int o = tid; o < per_pass * E; o += kThreads) {
          float sum = init;
          for (int t2 = 0; t2 < TG; ++t2)
            sum = pmax ? fmaxf(sum, red[t2 * per_pass * E + o]) : sum + red[t2 * per_pass * E + o];
          const int pr2 = p0 + o / E, r2 = pr2 / C16, d = (pr2 % C16) * E + o % E;
          float m = sum * scl;
          if (j > 0) m += qs[r2 * D + d];   // the same thread wrote it for the previous head
          qs[r2 * D + d] = m;
          if (last && row0 + r2 < nb) qbar[((int64_t)bh * nb + row0 + r2) * D + d] = m;
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float m = acc[e] * scl;
          if (j > 0) m += qs[r * D + c * E + e];
          qs[r * D + c * E + e] = m;
          if (last && row < nb) qbar[((int64_t)bh * nb + row) * D + c * E + e] = m;
        }
      }
    }
  }

  float acc[RW][CPL];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[r][c] = 0.f;

#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    __syncthreads();                        // previous chunk consumed (and qs written)
    {
      // all loads of the chunk first (up to 8 per thread: D <= 128), then the LDS stores
      constexpr int kMaxPer = 8;
      f32x4 vv[kMaxPer];
#pragma unroll
      for (int u = 0; u < kMaxPer; ++u) {
        const int e = tid + u * kThreads;
        vv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (e < 64 * D4) {
          const int col = e / D4, d4 = e - col * D4;
          const int j = c * 64 + col;
          if (j < nk) vv[u] = *(const f32x4*)(K + (int64_t)j * D + 4 * d4);
        }
      }
#pragma unroll
      for (int u = 0; u < kMaxPer; ++u) {
        const int e = tid + u * kThreads;
        if (e < 64 * D4) {
          const int col = e / D4, d4 = e - col * D4;
          float* dst = ks + col * KS + 4 * d4;
          dst[0] = vv[u][0]; dst[1] = vv[u][1]; dst[2] = vv[u][2]; dst[3] = vv[u][3];
        }
      }
    }
    __syncthreads();
    const float* qw = qs + wave * RW * D;
    const float* kr = ks + lane * KS;
    for (int d = 0; d < D; d += 4) {
      const float k0 = kr[d], k1 = kr[d + 1], k2 = kr[d + 2], k3 = kr[d + 3];
#pragma unroll
      for (int r = 0; r < RW; ++r) {
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
  for (int r = 0; r < RW; ++r) {
    const int row = row0 + wave * RW + r;
    if (row >= nb) break;                   // wave-uniform
    // columns past nk (and, causal, past the row) hold key 0, which no candidate (always
    // >= 1) and no T reached by the search (>= 1 once any bit is set) can count; causal rows
    // give their own block the largest key
    const int lim = causal ? row + 1 : nk;  // admissible columns j < lim
    const int kt = causal && row + 1 < topk ? row + 1 : topk;   // places of the row
    const int kr = kt - nrand;              // places taken by score (nrand = 0 if causal)
    uint32_t key[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = c * 64 + lane;
      key[c] = j < lim ? (causal && j == row ? 0xFFFFFFFFu : order_key(acc[r][c])) : 0u;
    }
    // chosen columns of this lane: the top kr by key (ties to the lower column) ...
    bool chosen[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) chosen[c] = false;
    if (kr > 0) {
      uint32_t T = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[c] >= cand));
        if (cnt >= kr) T = cand;
        if (cnt == kr) break;               // exactly kr keys >= T: T separates the top kr
      }
      int gt = 0;
#pragma unroll
      for (int c = 0; c < CPL; ++c) gt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[c] > T));
      const int need = kr - gt;             // places for keys equal to T
      int eq_before = 0;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const bool valid = (c * 64 + lane) < lim;
        const bool is_eq = valid && key[c] == T;
        const uint64_t meq = __builtin_amdgcn_ballot_w64(is_eq);
        chosen[c] = valid && (key[c] > T || (is_eq && eq_before + lanes_below(meq) < need));
        eq_before += __builtin_popcountll(meq);
      }
    }
    // ... then nrand random others, one draw at a time (uniform across the wave)
    if (nrand > 0) {
      const uint64_t srow = (uint64_t)((int64_t)sh * nb + row);
      for (int p = 0; p < nrand; ++p) {
        const uint32_t m = (uint32_t)(nk - kr - p);              // blocks not yet chosen
        const uint32_t x = (uint32_t)(splitmix64(seed, srow * 65536u + (uint64_t)p) % m);
        uint32_t before = 0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const uint64_t mrem = __builtin_amdgcn_ballot_w64((c * 64 + lane) < nk && !chosen[c]);
          const uint32_t cnt = (uint32_t)__builtin_popcountll(mrem);
          if (x >= before && x < before + cnt && ((mrem >> lane) & 1ull) &&
              (uint32_t)lanes_below(mrem) == x - before)
            chosen[c] = true;
          before += cnt;
        }
      }
    }
    for (int j = 0; j < nh; ++j) {
      int32_t* out = idx + ((int64_t)(bh + j) * nb + row) * topk;
      int sel_before = 0;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const uint64_t msel = __builtin_amdgcn_ballot_w64(chosen[c]);
        if (chosen[c]) out[sel_before + lanes_below(msel)] = c * 64 + lane;
        sel_before += __builtin_popcountll(msel);
      }
      for (int p = kt + lane; p < topk; p += kWave) out[p] = -1;   // unused causal places
    }
  }
}

template <int KIND, int CPL>
hipError_t launch(int64_t B, int64_t N, int Hq, int Hkv, int nb, int nk, int D, int block,
                  int topk, const void* q, float* qbar, const float* kbar, int32_t* idx,
                  unsigned flags, int nrand, uint64_t seed, hipStream_t stream) {
  constexpr int RG = SelCfg<CPL>::RG;
  const int row_tiles = (nb + RG - 1) / RG;
  const int HS = (flags & kGroup) ? Hkv : Hq;
  const dim3 grid((unsigned)(B * HS * row_tiles));
  const size_t lds = (size_t)(64 * (D + 1) + RG * D) * sizeof(float);
  select_kernel<KIND, CPL><<<grid, kThreads, lds, stream>>>(
      (const uint8_t*)q, qbar, kbar, idx, N, Hq, Hkv, nb, nk, D, block, topk, row_tiles,
      1.0f / (float)block, flags, nrand, seed);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(int64_t B, int64_t N, int Hq, int Hkv, int nb, int nk, int D, int block,
                       int topk, const void* q, float* qbar, const float* kbar, int32_t* idx,
                       unsigned flags, int nrand, uint64_t seed, hipStream_t stream) {
#define BSATTN_SELECT_CPL(cpl) \
  launch<KIND, cpl>(B, N, Hq, Hkv, nb, nk, D, block, topk, q, qbar, kbar, idx, flags, nrand, seed, stream)
  if (nk <= 64) return BSATTN_SELECT_CPL(1);
  if (nk <= 128) return BSATTN_SELECT_CPL(2);
  if (nk <= 256) return BSATTN_SELECT_CPL(4);
  if (nk <= 512) return BSATTN_SELECT_CPL(8);
  return BSATTN_SELECT_CPL(16);
#undef BSATTN_SELECT_CPL
}

}  // namespace

hipError_t launch_pool_score_select(int kind, int64_t B, int64_t N, int Hq, int Hkv, int D,
                                    int block, int topk, int64_t nkb, const void* q, float* qbar,
                                    const float* kbar, int32_t* idx, unsigned flags,
                                    int nrand, uint64_t seed, hipStream_t stream) {
  const int nb = (int)(N / block), nk = (int)nkb;
  if (kind == 0) return launch_kind<0>(B, N, Hq, Hkv, nb, nk, D, block, topk, q, qbar, kbar, idx, flags, nrand, seed, stream);
  if (kind == 1) return launch_kind<1>(B, N, Hq, Hkv, nb, nk, D, block, topk, q, qbar, kbar, idx, flags, nrand, seed, stream);
  return launch_kind<2>(B, N, Hq, Hkv, nb, nk, D, block, topk, q, qbar, kbar, idx, flags, nrand, seed, stream);
}

}  // namespace bsattn
