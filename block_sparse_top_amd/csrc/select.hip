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
// Layout: one work-group = 4 waves = 16 consecutive query-block rows of one (batch, query
// head). It first averages its rows' query tokens (16-byte loads, streamed past the caches:
// this phase is HBM-bound and overlaps the arithmetic of the other work-groups on the CU),
// keeps the pooled rows in LDS and also stores them to the workspace. Key-block columns are
// staged through LDS 64 at a time with coalesced row loads; the block scores of a chunk are
// a 16 x 64 product on the bf16 MFMA with fp32 accuracy (three-part bf16 splits of the fp32
// operands; the MSA page's scores as a matrix product), the same arithmetic for every column
// (equal pooled key blocks give equal scores). Each wave then holds 4 rows x CPL columns of scores in registers, lane l owning
// columns j = l + 64*c.
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

// A work-group takes RG = 16 query-block rows (one 16-row tile of the fp32 MFMA; 4 waves) or,
// from 512 key blocks on, 32 rows (8 waves): every work-group streams all pooled keys through
// LDS, and 32 rows halve that traffic. 4 rows per wave for the selection.
// LDS floats of the pooled query rows ([RG][D] fp32); at D = 128 the same space then holds
// their three bf16 parts ([3][RG] rows of 2D + 16 bytes: 16 rows of a read on distinct banks)
constexpr int kQPartRow = 2 * 128 + 16;
constexpr int query_lds_floats(int RG, int D) {
  return D == 128 ? 3 * RG * kQPartRow / 4 : RG * D;
}

template <int CPL>
struct SelCfg {
  static constexpr int NWV = CPL >= 8 ? 8 : 4;                 // waves
  static constexpr int NT = NWV * kWave;                       // threads
  static constexpr int RW = 4;                                 // rows per wave
  static constexpr int RG = NWV * RW;                          // rows per work-group
};

// storage kind; score columns per lane: nk <= 64 * CPL; head dimension
template <int KIND, int CPL, int D>
__global__ __launch_bounds__(SelCfg<CPL>::NT) void select_kernel(
    const uint8_t* __restrict__ q, float* __restrict__ qbar, const float* __restrict__ kbar,
    int32_t* __restrict__ idx, int64_t N, int Hq, int Hkv, int nb, int nk, int block,
    int topk, int row_tiles, float inv_block, unsigned flags, int nrand, uint64_t seed,
    int D_rt) {
  constexpr int RW = SelCfg<CPL>::RW, RG = SelCfg<CPL>::RG, kThreads = SelCfg<CPL>::NT;
  constexpr int E = Vec<KIND>::E;
  constexpr int EB = 16 / E;                // bytes per stored element
  extern __shared__ float smem[];
  constexpr int KS = D + 4;                 // padded row stride of the key chunk (16-byte rows)
  constexpr int SS = 64 + 4;                // row stride of the score chunk
  float* ks = smem;                         // [64][D+4] current key-block chunk
  constexpr int kRed = RG * (D / E) < kThreads ? kThreads * E : 0;   // pooling partial sums
  float* qs = smem + (64 * KS > kRed ? 64 * KS : kRed);   // [RG][D] pooled query rows
  float* sc = qs + query_lds_floats(RG, D);  // [RG][64+4] score chunk (MFMA tiles -> rows)

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
  constexpr int D4 = D / 4;

  // ---- pool the RG query rows: pair (row r, 16-byte column c); TG token groups per pair.
  // (This phase takes the head dimension as a run-time value: with the constant the compiler
  // unrolls it into many more live registers, fewer work-groups per CU and a slower stream.)
  const int Dr = D_rt;
  const float init = pmax ? -__builtin_inff() : 0.f;
  const float scl = pmax ? 1.f : inv_block;
  for (int j = 0; j < nh; ++j) {
    const int h = h0 + j;
    const bool last = j == nh - 1;
    const int C16 = Dr / E;                  // 16-byte columns per token of one head
    const int pairs = RG * C16;
    const int per_pass = pairs < kThreads ? pairs : kThreads;
    const int TG = kThreads / per_pass;     // token groups (>= 1)
    const int64_t tok_bytes = (int64_t)Hq * Dr * EB;
    float* red = ks;                        // [TG][per_pass][E] partial sums (fits: D >= 64)
    for (int p0 = 0; p0 < pairs; p0 += per_pass) {
      const int pr = p0 + tid % per_pass, tg = tid / per_pass;
      const int r = pr / C16, c = pr % C16;
      const int row = row0 + r;
      float acc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = init;
      if (tg < TG && row < nb) {
        const uint8_t* src = q + (((int64_t)b * N + (int64_t)row * block) * Hq + h) * Dr * EB + c * 16;
        int t = tg;
        // loads in flight per thread: 16 at D = 128 (bf16/fp32: 5 % faster on 128-token
        // blocks), 8 otherwise (16 was 2.6 % slower at D = 64: fewer work-groups per CU)
        constexpr int UQ = D == 128 && KIND != 2 ? 16 : 8;
        for (; t + (UQ - 1) * TG < block; t += UQ * TG) {
          u32x4 w[UQ];
#pragma unroll
          for (int u = 0; u < UQ; ++u)
            w[u] = __builtin_nontemporal_load((const u32x4*)(src + (int64_t)(t + u * TG) * tok_bytes));
          if (pmax) {
#pragma unroll
            for (int u = 0; u < UQ; ++u) Vec<KIND>::vmax(w[u], acc);
          } else {
#pragma unroll
            for (int u = 0; u < UQ; ++u) Vec<KIND>::add(w[u], acc);
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
          if (j > 0) m += qs[r2 * Dr + d];   // the same thread wrote it for the previous head
          qs[r2 * Dr + d] = m;
          if (last && row0 + r2 < nb) qbar[((int64_t)bh * nb + row0 + r2) * Dr + d] = m;
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float m = acc[e] * scl;
          if (j > 0) m += qs[r * Dr + c * E + e];
          qs[r * Dr + c * E + e] = m;
          if (last && row < nb) qbar[((int64_t)bh * nb + row) * Dr + c * E + e] = m;
        }
      }
    }
  }

  // ---- scores with fp32 accuracy on the bf16 MFMA (v_mfma_f32_16x16x32_bf16): every fp32
  // operand value x is split into three bf16 parts x = x0 + x1 + x2 (x0 = bf16(x),
  // x1 = bf16(x - x0), x2 = x - x0 - x1; exact for normal values) and a score is
  // q0.k0 + (q0.k1 + q1.k0 + q0.k2 + q1.k1 + q2.k0): products of bf16 parts are exact in fp32,
  // the three products left out are below 2^-23 of sum_d |q_d k_d|, and the six bf16
  // products take 3/8 of the fp32 MFMA's time (the MSA page's scores as a matrix product).
  // Per 64-column chunk each wave forms the 16 x 16 tile S[rows][16*(wave%4) .. +16) = qs K^T;
  // the k-slot group q4 = lane / 16 of a lane carries d = 32s + 8*q4 .. +7 at k-step s on both
  // operands. The query parts are formed once; the key values are split as they are read
  // from the fp32 chunk in LDS. Every score goes through the same products and sums in the
  // same order, so equal pooled key blocks give equal scores. The tile goes through LDS (sc)
  // to the selection layout, lane = column, 4 rows per wave.
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  const int m16 = lane & 15, q4 = lane >> 4;
  constexpr int NK = D / 32;                // k-steps per tile (2 or 4)
  auto split8 = [](const f32x4v& lo4, const f32x4v& hi4, bf16x8 part[3]) {
    // three bf16 parts of 8 consecutive values (part p: x_p of each value, in order)
    uint32_t w[3][4];
    const f32x4v v2[2] = {lo4, hi4};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float a = v2[h][2 * e], b = v2[h][2 * e + 1];
        const uint32_t p0 = pack_bf16x2(a, b);
        const float ra = a - bf16lo(p0), rb = b - bf16hi(p0);
        const uint32_t p1 = pack_bf16x2(ra, rb);
        w[0][2 * h + e] = p0;
        w[1][2 * h + e] = p1;
        w[2][2 * h + e] = pack_bf16x2(ra - bf16lo(p1), rb - bf16hi(p1));
      }
#pragma unroll
    for (int p = 0; p < 3; ++p)
      part[p] = __builtin_bit_cast(bf16x8, u32x4{w[p][0], w[p][1], w[p][2], w[p][3]});
  };
  // A operands (qs[m16][32s + 8*q4 .. +7], split): in registers at D = 64; at D = 128 in LDS
  // (the parts overwrite qs), read per k-step, which keeps 1024 key blocks at 4 waves per SIMD
  bf16x8 qa[D == 64 ? NK : 1][3];
  char* qp = (char*)qs;                     // D = 128: [3][RG][kQPartRow bytes]
  __syncthreads();                          // qs complete
  if constexpr (D == 64) {
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const float* qrow = qs + (16 * (wave >> 2) + m16) * D + 32 * s + 8 * q4;
      split8(*(const f32x4v*)qrow, *(const f32x4v*)(qrow + 4), qa[s]);
    }
  } else {
    static_assert(RG * D / 8 == kThreads, "one group of 8 pooled values per thread");
    const int r = tid / (D / 8), c8 = tid % (D / 8);
    const float* src = qs + r * D + 8 * c8;
    bf16x8 part[3];
    split8(*(const f32x4v*)src, *(const f32x4v*)(src + 4), part);
    __syncthreads();                        // every thread has read its values of qs
#pragma unroll
    for (int p = 0; p < 3; ++p)
      *(bf16x8*)(qp + (p * RG + r) * kQPartRow + 16 * c8) = part[p];
    __syncthreads();
  }
  float acc[RW][CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    // causal: a chunk that starts past the work-group's last row holds no admissible column
    // of its rows (all keys 0 below), nor does any later one; the test is the same for the
    // whole work-group, so every barrier is still reached by all its waves or by none
    if (causal && c * 64 > row0 + RG - 1) {
#pragma unroll
      for (int r = 0; r < RW; ++r) acc[r][c] = 0.f;
      continue;
    }
    __syncthreads();                        // previous chunk's ks and sc consumed
    {
      // all loads of the chunk first (up to 8 per thread: D <= 128), then the LDS stores
      // (columns past nk load the last key block and are zeroed after the load)
      constexpr int kPer = 64 * D4 / kThreads;   // 4 (D = 64) or 8 (D = 128)
      f32x4 vv[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int e = tid + u * kThreads;
        const int col = e / D4, d4 = e - col * D4;
        const int j = c * 64 + col;
        vv[u] = *(const f32x4*)(K + (int64_t)(j < nk ? j : nk - 1) * D + 4 * d4);
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int e = tid + u * kThreads;
        const int col = e / D4, d4 = e - col * D4;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        *(f32x4*)(ks + col * KS + 4 * d4) = c * 64 + col < nk ? vv[u] : z;
      }
    }
    __syncthreads();
    {
      // the leading product in hi, the five smaller ones in two chains (lo0, lo1), added at
      // the end in a fixed order: the same for every column
      const int ct = wave & 3;              // column tile of this wave (16 columns)
      const float* kb = ks + (16 * ct + m16) * KS + 8 * q4;
      f32x4v hi = {0.f, 0.f, 0.f, 0.f}, lo0 = hi, lo1 = hi;
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        bf16x8 kp[3], qv[3];
        split8(*(const f32x4v*)(kb + 32 * s), *(const f32x4v*)(kb + 32 * s + 4), kp);
        if constexpr (D == 64) {
#pragma unroll
          for (int p = 0; p < 3; ++p) qv[p] = qa[s][p];
        } else {
#pragma unroll
          for (int p = 0; p < 3; ++p)
            qv[p] = *(const bf16x8*)(qp + (p * RG + 16 * (wave >> 2) + m16) * kQPartRow +
                                     2 * (32 * s + 8 * q4));
        }
        hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qv[0], kp[0], hi, 0, 0, 0);
        lo0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qv[0], kp[1], lo0, 0, 0, 0);
        lo1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qv[1], kp[0], lo1, 0, 0, 0);
        lo0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qv[0], kp[2], lo0, 0, 0, 0);
        lo1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qv[1], kp[1], lo1, 0, 0, 0);
        lo0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qv[2], kp[0], lo0, 0, 0, 0);
      }
      const f32x4v t = hi + (lo0 + lo1);
      // lane holds S[row 16*(wave/4) + 4*q4 + e][column 16*(wave%4) + m16]
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[(16 * (wave >> 2) + 4 * q4 + e) * SS + 16 * ct + m16] = t[e];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RW; ++r) acc[r][c] = sc[(wave * RW + r) * SS + lane];
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

template <int KIND, int CPL, int D>
hipError_t launch(int64_t B, int64_t N, int Hq, int Hkv, int nb, int nk, int block,
                  int topk, const void* q, float* qbar, const float* kbar, int32_t* idx,
                  unsigned flags, int nrand, uint64_t seed, hipStream_t stream) {
  constexpr int RG = SelCfg<CPL>::RG, NT = SelCfg<CPL>::NT;
  const int row_tiles = (nb + RG - 1) / RG;
  const int HS = (flags & kGroup) ? Hkv : Hq;
  const dim3 grid((unsigned)(B * HS * row_tiles));
  // the key chunk's LDS also holds the pooling phase's partial sums (TG x pairs x E floats)
  constexpr int E = Vec<KIND>::E;
  constexpr int pairs = RG * (D / E);
  constexpr int red = pairs < NT ? NT * E : 0;    // as the kernel reserves it
  constexpr int kchunk = 64 * (D + 4) > red ? 64 * (D + 4) : red;
  const size_t lds = (size_t)(kchunk + query_lds_floats(RG, D) + RG * (64 + 4)) * sizeof(float);
  select_kernel<KIND, CPL, D><<<grid, NT, lds, stream>>>(
      (const uint8_t*)q, qbar, kbar, idx, N, Hq, Hkv, nb, nk, block, topk, row_tiles,
      1.0f / (float)block, flags, nrand, seed, D);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(int64_t B, int64_t N, int Hq, int Hkv, int nb, int nk, int D, int block,
                       int topk, const void* q, float* qbar, const float* kbar, int32_t* idx,
                       unsigned flags, int nrand, uint64_t seed, hipStream_t stream) {
#define BSATTN_SELECT_CPL(cpl)                                                                  \
  (D == 64 ? launch<KIND, cpl, 64>(B, N, Hq, Hkv, nb, nk, block, topk, q, qbar, kbar, idx, flags, \
                                   nrand, seed, stream)                                          \
           : launch<KIND, cpl, 128>(B, N, Hq, Hkv, nb, nk, block, topk, q, qbar, kbar, idx,      \
                                    flags, nrand, seed, stream))
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
