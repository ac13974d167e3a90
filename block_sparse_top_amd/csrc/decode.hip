// Decode step: one new query token per sequence against a KV cache, with the pooled key
// blocks of the cache kept up to date as blocks complete.
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"), "SparseFormer
// 注意力实现": mean-pooled key blocks, top-k blocks by the product with the (here single-token)
// query, attention over the chosen blocks with scale 1/sqrt(D). MSA page
// ("从M2.7到M3：多模态模型稀疏注意力架构设计与实现全解析") §5.2: first-token latency comes from
// an unoptimised block-scoring step. Step rule for a sequence of L cached tokens (the query is
// token L-1): its own block (L-1)/b is always used; the other min(k, own+1) - 1 places go to
// the complete blocks j < own with the largest q . kbar_j (ties to the lower j).
//
// Kernels (bf16 caches [B, Lmax, Hkv, D]; fp32 pooled cache stored transposed,
// [B, Hkv, D, Lmax/b], so that lanes owning consecutive blocks read consecutive words):
//   pool_new_kernel    one work-group per (sequence, block): pools the blocks completed
//                      between the old and the new length (all complete blocks without old
//                      lengths).
//   dselect_kernel     one work-group of 4 waves per (sequence, query head) for up to 2048
//                      blocks (one wave beyond; with a group-shared selection per (sequence,
//                      KV head), on the sum of the group's queries, writing the same row for
//                      each of its query heads): lane l owns blocks l + 64c; each wave sums a
//                      quarter of d in order (coalesced loads of the transposed cache), the
//                      quarters meet in LDS in a fixed order (fp32 scores), then one wave runs
//                      the prefill selection's bitwise threshold search with ballots and
//                      compacts the chosen blocks in ascending order.
//   dattn_kernel       split-K over the chosen blocks (flash-decoding): one wave per
//                      (sequence, query head, split), the G heads of a KV head side by side;
//                      per block, groups of D/8 lanes read key rows together for the scores
//                      (16-byte loads, partial dots summed across the group), the weights go
//                      through LDS, then groups of lanes
//                      own 8 consecutive d of one key (16-byte loads, several keys in
//                      flight) for the weighted value sum. Writes the split's (max, sum,
//                      unnormalised output).
//   dcombine_kernel    per (sequence, query head): merges the splits, writes bf16.
// The work is HBM-bound (each key and value of a chosen block is read once per query head);
// the single query row leaves nothing for the matrix cores.
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------- pooling of new blocks
__global__ __launch_bounds__(256) void pool_new_kernel(const uint16_t* __restrict__ kc,
                                                       const int32_t* __restrict__ lens_old,
                                                       const int32_t* __restrict__ lens_new,
                                                       float* __restrict__ kbar, int64_t Lmax,
                                                       int Hkv, int D, int block, int nbmax) {
  const int b = blockIdx.y, j = blockIdx.x;
  const int64_t Ln = lens_new[b];
  const int64_t Lo = lens_old ? lens_old[b] : 0;
  if (Ln < 1 || Ln > Lmax || Lo < 0 || Lo > Ln) return;
  if (j < Lo / block || j >= Ln / block) return;
  const int V = Hkv * D / 8;                            // 16-byte chunks per token row
  const int64_t rs = (int64_t)Hkv * D;
  const float inv = 1.0f / (float)block;
  for (int c = threadIdx.x; c < V; c += blockDim.x) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const uint16_t* p = kc + ((int64_t)b * Lmax + (int64_t)j * block) * rs + 8 * c;
    for (int t = 0; t < block; ++t) Vec<1>::add(*(const u32x4*)(p + t * rs), acc);
    const int g = (8 * c) / D, d0 = (8 * c) % D;
    float* o = kbar + (((int64_t)b * Hkv + g) * D + d0) * nbmax + j;   // [.., d, j]
#pragma unroll
    for (int e = 0; e < 8; ++e) o[(int64_t)e * nbmax] = acc[e] * inv;
  }
}

// whole-wave reductions: the DPP steps within each 16 lanes, then across 16 and 32 lanes
__device__ __forceinline__ float wave_sum(float a) {
  a = group_sum<16>(a);
  a += __shfl_xor(a, 16);
  return a + __shfl_xor(a, 32);
}
__device__ __forceinline__ float wave_max(float a) {
  a = fmaxf(a, dpp_mov<kDppXor1>(a));
  a = fmaxf(a, dpp_mov<kDppXor2>(a));
  a = fmaxf(a, dpp_mov<kDppHalfMirror>(a));
  a = fmaxf(a, dpp_mov<kDppMirror>(a));
  a = fmaxf(a, __shfl_xor(a, 16));
  return fmaxf(a, __shfl_xor(a, 32));
}

// ---------------------------------------------------------------- selection
constexpr int kSelWaves = 4;                  // (sequence, head) pairs per work-group
constexpr int kMaxDecodeGroup = 16;           // query heads per KV head in one work-group
constexpr int kSelCols = kMaxDecodeBlocks / kWave;   // blocks per lane: nb <= 8192

// SPLIT waves per (sequence, head) share the d range (SPLIT = 4, nb <= 2048) or one wave does
// all of it (SPLIT = 1, kSelWaves heads per work-group)
template <int D, int CPL, int SPLIT>
__global__ __launch_bounds__(256) void dselect_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ kbar,
    const int32_t* __restrict__ lens, int32_t* __restrict__ idx, int64_t Lmax, int Hq, int Hkv,
    int block, int nbmax, int topk, int heads, bool group) {
  constexpr int HPW = SPLIT == 1 ? kSelWaves : 1;       // (sequence, head) pairs per group
  __shared__ float qs[HPW][D];
  __shared__ float partial[SPLIT == 1 ? 1 : SPLIT - 1][SPLIT == 1 ? 1 : 64 * CPL];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int slot = SPLIT == 1 ? wave : 0;               // this wave's pair in the group
  const int part = SPLIT == 1 ? 0 : wave;               // this wave's quarter of d
  const int bh = blockIdx.x * HPW + slot;
  if (bh >= heads) return;                    // SPLIT == 1 only (grid covers heads exactly
                                              // for SPLIT == 4): no barrier follows
  // selection row bh = b * HS + s: query head s, or (group) KV head s, whose G query heads'
  // queries are summed (in head order) and which writes the same row for each of them
  const int G = Hq / Hkv, HS = group ? Hkv : Hq;
  const int b = bh / HS, s = bh % HS;
  const int g = group ? s : s / G;
  const int h0 = group ? s * G : s, nh = group ? G : 1;
  int32_t* out = idx + ((int64_t)b * Hq + h0) * topk;     // rows out + j * topk, j < nh
  const int64_t L = lens[b];
  const bool len_ok = L >= 1 && L <= Lmax;
  const int own = len_ok ? (int)((L - 1) / block) : 0;
  const int kb = own + 1 < topk ? own + 1 : topk;
  const int need = len_ok ? kb - 1 : 0;       // places for complete earlier blocks
  for (int d = lane; d < D; d += kWave) {
    const uint16_t* qh = q + ((int64_t)b * Hq + h0) * D + d;
    float x = __uint_as_float((uint32_t)qh[0] << 16);
    for (int j = 1; j < nh; ++j) x += __uint_as_float((uint32_t)qh[(int64_t)j * D] << 16);
    qs[slot][d] = x;
  }
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  if (need > 0) {
    // scores: lane owns blocks lane + 64c (c < CPL); this wave's d range in order
    const float* K = kbar + ((int64_t)b * Hkv + g) * D * nbmax;
    constexpr int DR = D / SPLIT;
    // d rows loaded before their products: 64 values per lane in flight (RB * CPL <= 64)
    constexpr int RB0 = CPL >= 64 ? 1 : 64 / CPL;
    constexpr int RB = RB0 < DR ? RB0 : DR;
    static_assert(DR % RB == 0, "d range in whole row batches");
    // the loads of RB rows are all issued before the first product, so their latencies
    // overlap (a dependent load-then-use per row leaves the wave waiting on every row);
    // the products keep ascending d, so the sums are unchanged
    for (int d0 = part * DR; d0 < (part + 1) * DR; d0 += RB) {
      float kv[RB][CPL];
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int j = lane + 64 * c;
          kv[u][c] = j < own ? K[(int64_t)(d0 + u) * nbmax + j] : 0.f;
        }
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const float qd = qs[slot][d0 + u];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          if (lane + 64 * c < own) acc[c] = __builtin_fmaf(qd, kv[u][c], acc[c]);
      }
    }
  }
  if (SPLIT > 1) {                            // quarters 1.. to LDS, wave 0 adds them in order
    if (part > 0)
#pragma unroll
      for (int c = 0; c < CPL; ++c) partial[part - 1][lane + 64 * c] = acc[c];
    __syncthreads();
    if (part > 0) return;
#pragma unroll
    for (int w = 0; w < SPLIT - 1; ++w)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] += partial[w][lane + 64 * c];
  }
  if (!len_ok) {                              // invalid length: no block
    for (int j = 0; j < nh; ++j)
      for (int p = lane; p < topk; p += kWave) out[(int64_t)j * topk + p] = -1;
    return;
  }
  if (need > 0) {
    uint32_t key[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) key[c] = (lane + 64 * c) < own ? order_key(acc[c]) : 0u;
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int c = 0; c < CPL; ++c) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[c] >= cand));
      if (cnt >= need) T = cand;
      if (cnt == need) break;
    }
    int gt = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) gt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[c] > T));
    const int eq_need = need - gt;
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const bool valid = (lane + 64 * c) < own;
      const bool is_eq = valid && key[c] == T;
      const uint64_t meq = __builtin_amdgcn_ballot_w64(is_eq);
      const bool sel = valid && (key[c] > T || (is_eq && eq_before + lanes_below(meq) < eq_need));
      const uint64_t msel = __builtin_amdgcn_ballot_w64(sel);
      if (sel)
        for (int j = 0; j < nh; ++j) out[(int64_t)j * topk + sel_before + lanes_below(msel)] = lane + 64 * c;
      eq_before += __builtin_popcountll(meq);
      sel_before += __builtin_popcountll(msel);
    }
  }
  for (int j = 0; j < nh; ++j) {
    if (lane == 0) out[(int64_t)j * topk + kb - 1] = own;
    for (int p = kb + lane; p < topk; p += kWave) out[(int64_t)j * topk + p] = -1;
  }
}

// ---------------------------------------------------------------- split-K attention
template <int D>
__global__ __launch_bounds__(64) void dattn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ lens, float* __restrict__ part, int64_t Lmax, int Hq, int Hkv,
    int block, int topk, int splits, float c) {
  __shared__ float qs[D];
  __shared__ float ps[128];                   // weights of one block (block <= 128)
  // work order (b, KV head, split, head within group): the G query heads of a KV head that
  // read the same split of their blocks run side by side on one XCD (under a group-shared
  // selection they read the same keys and values, which then come from its L2)
  const int G = Hq / Hkv;
  uint32_t w = xcd_remap(blockIdx.x, gridDim.x);
  const int hh = (int)(w % G);
  w /= G;
  const int sp = (int)(w % splits);
  w /= splits;
  const int g = (int)(w % Hkv), b = (int)(w / Hkv);
  const int h = g * G + hh;
  const int bh = b * Hq + h;
  const int lane = threadIdx.x;
  const int64_t L = lens[b];
  const int64_t rs = (int64_t)Hkv * D;
  float* my = part + ((int64_t)bh * splits + sp) * (D + 2);
  for (int d = lane; d < D; d += 64) {
    const uint16_t w = q[(int64_t)bh * D + d];
    qs[d] = __uint_as_float((uint32_t)w << 16);
  }
  __syncthreads();
  const int32_t* row = idx + (int64_t)bh * topk;
  const int per = (topk + splits - 1) / splits;
  const int e0 = sp * per, e1 = e0 + per < topk ? e0 + per : topk;
  float m = -__builtin_inff(), l = 0.f;
  // value accumulators: lane owns d = 8*dg .. 8*dg+7 of keys kq, kq + KG, ... (KG key groups
  // of LG lanes; the groups are summed at the end)
  constexpr int LG = D / 8, KG = 64 / LG;
  const int dg = lane % LG, kq = lane / LG;
  float o[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) o[x] = 0.f;
  const uint16_t* kb0 = kc + (int64_t)b * Lmax * rs + (int64_t)g * D;
  const uint16_t* vb0 = vc + (int64_t)b * Lmax * rs + (int64_t)g * D;
  const bool len_ok = L >= 1 && L <= Lmax;
  float qv[8];                                // q[8*dg .. 8*dg+7] for the score pass
#pragma unroll
  for (int x = 0; x < 8; ++x) qv[x] = qs[8 * dg + x];
  for (int e = e0; e < e1 && len_ok; ++e) {
    const int j = row[e];
    if (j < 0 || (int64_t)j * block >= L) continue;   // unused place or beyond the cache
    const int64_t t0 = (int64_t)j * block;
    const int nk = (int)(L - t0 < block ? L - t0 : block);   // own block: tokens < L
    // scores: the LG lanes of key group kq read one key row together (16 bytes each, so one
    // load instruction covers KG whole rows), multiply by their 8 query values and add the
    // partial sums across the group; four rounds of keys are in flight
    __syncthreads();                          // previous block done with ps
    for (int t = kq; t < nk; t += 4 * KG) {
      u32x4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int tt = t + u * KG;
        w[u] = u32x4{0u, 0u, 0u, 0u};
        if (tt < nk) w[u] = *(const u32x4*)(kb0 + (t0 + tt) * rs + 8 * dg);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float a = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          a = __builtin_fmaf(qv[2 * x], bf16lo(w[u][x]), a);
          a = __builtin_fmaf(qv[2 * x + 1], bf16hi(w[u][x]), a);
        }
        a = group_sum<LG>(a);
        const int tt = t + u * KG;
        if (dg == 0 && tt < nk) ps[tt] = a * c;   // exp2 domain
      }
    }
    __syncthreads();
    float s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = lane + 64 * u;
      s[u] = t < nk ? ps[t] : -__builtin_inff();
    }
    float mb = fmaxf(s[0], s[1]);
    mb = wave_max(mb);
    const float mn = fmaxf(m, mb);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);    // 0 on the first block
    m = mn;
    float lp = 0.f;
    __syncthreads();                          // scores read before the weights replace them
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = lane + 64 * u;
      const float p = t < nk ? __builtin_amdgcn_exp2f(s[u] - m) : 0.f;
      if (t < block) ps[t] = p;
      lp += p;
    }
    lp = wave_sum(lp);
    l = l * alpha + lp;
#pragma unroll
    for (int x = 0; x < 8; ++x) o[x] *= alpha;
    __syncthreads();
    const uint16_t* vrow = vb0 + (t0 + kq) * rs + 8 * dg;
    int t = kq;
    for (; t + 3 * KG < nk; t += 4 * KG) {    // four keys of this lane in flight
      u32x4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = *(const u32x4*)(vrow + (int64_t)(t - kq + u * KG) * rs);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float p = ps[t + u * KG];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          o[2 * x] = __builtin_fmaf(p, bf16lo(w[u][x]), o[2 * x]);
          o[2 * x + 1] = __builtin_fmaf(p, bf16hi(w[u][x]), o[2 * x + 1]);
        }
      }
    }
    for (; t < nk; t += KG) {
      const u32x4 w = *(const u32x4*)(vrow + (int64_t)(t - kq) * rs);
      const float p = ps[t];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        o[2 * x] = __builtin_fmaf(p, bf16lo(w[x]), o[2 * x]);
        o[2 * x + 1] = __builtin_fmaf(p, bf16hi(w[x]), o[2 * x + 1]);
      }
    }
  }
  // sum the key groups (lanes dg, dg + LG, ...)
#pragma unroll
  for (int off = LG; off < 64; off <<= 1)
#pragma unroll
    for (int x = 0; x < 8; ++x) o[x] += __shfl_xor(o[x], off);
  if (kq == 0) {
#pragma unroll
    for (int x = 0; x < 8; ++x) my[2 + 8 * dg + x] = o[x];
  }
  if (lane == 0) {
    my[0] = m;
    my[1] = l;
  }
}

// Group-shared selection: one work-group of G waves per (sequence, KV head, split), wave w
// computing query head g*G + w over the group's common blocks. Each block's keys and values
// go into LDS once for all G waves (the per-head kernel would read them G times); the score
// pass (groups of D/8 lanes per key row, partial dots summed across the group), the weights
// and the value pass then run per wave from LDS, writing the same partial results as
// dattn_kernel for dcombine_kernel.
// The tiles move with global_load_lds_dwordx4 (1 KiB of consecutive rows per wave
// instruction, the instructions of a tile dealt round-robin over the waves) and overlap the
// arithmetic: the next block's keys start as soon as every wave has scored the current keys,
// its values as soon as every wave has summed the current values. Every wave issues the same
// number of transfers per tile (a wave short of a distinct one repeats the tile's last: the
// same bytes to the same place), so the waits count a fixed number per tile.

// vmcnt-only waits (expcnt and lgkmcnt left free), gfx9 s_waitcnt encoding
template <int N>
__device__ __forceinline__ void dwait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// wait until at most n of this wave's vector-memory operations are in flight (n uniform)
__device__ __forceinline__ void dwait_vmcnt_le(int n) {
  switch (n) {
    case 0: dwait_vmcnt<0>(); break;
    case 1: dwait_vmcnt<1>(); break;
    case 2: dwait_vmcnt<2>(); break;
    case 3: dwait_vmcnt<3>(); break;
    case 4: dwait_vmcnt<4>(); break;
    case 5: dwait_vmcnt<5>(); break;
    case 6: dwait_vmcnt<6>(); break;
    case 7: dwait_vmcnt<7>(); break;
    case 8: dwait_vmcnt<8>(); break;
    default: dwait_vmcnt<0>(); break;         // (more per tile: wait for all, still correct)
  }
}

template <int D>
__global__ __launch_bounds__(1024) void dattn_group_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ lens, float* __restrict__ part, int64_t Lmax, int Hq, int Hkv,
    int block, int topk, int splits, float c) {
  constexpr int CH = D / 8;                   // 16-byte chunks per key row
  // LDS (sized at launch): K and V rows of one block [block][D] bf16, the G queries [G][D] and
  // weights [G][block] fp32
  extern __shared__ __attribute__((aligned(1024))) char dsm[];
  const int G = Hq / Hkv;
  uint16_t* Ks = (uint16_t*)dsm;
  uint16_t* Vs = Ks + block * D;
  float* qsm = (float*)(Vs + block * D);
  float* psm = qsm + G * D;
  uint32_t w = xcd_remap(blockIdx.x, gridDim.x);   // (b, KV head, split)
  const int sp = (int)(w % splits);
  w /= splits;
  const int g = (int)(w % Hkv), b = (int)(w / Hkv);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int h = g * G + wave, bh = b * Hq + h;
  const int64_t L = lens[b];
  const int64_t rs = (int64_t)Hkv * D;
  float* my = part + ((int64_t)bh * splits + sp) * (D + 2);
  for (int d = lane; d < D; d += kWave)
    qsm[wave * D + d] = __uint_as_float((uint32_t)q[(int64_t)bh * D + d] << 16);
  const int32_t* row = idx + ((int64_t)b * Hq + g * G) * topk;   // the group's common row
  const int per = (topk + splits - 1) / splits;
  const int e0 = sp * per, e1 = e0 + per < topk ? e0 + per : topk;
  float m = -__builtin_inff(), l = 0.f;
  constexpr int LG = D / 8, KG = 64 / LG;
  const int dg = lane % LG, kq = lane / LG;
  float o[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) o[x] = 0.f;
  const uint16_t* kb0 = kc + (int64_t)b * Lmax * rs + (int64_t)g * D;
  const uint16_t* vb0 = vc + (int64_t)b * Lmax * rs + (int64_t)g * D;
  const bool len_ok = L >= 1 && L <= Lmax;
  // transfers: a tile is block*CH/64 wave instructions of 1 KiB; wave w issues ni of them
  // (instructions w, w+G, ...; the last one repeated where a wave runs out)
  const int nins = block * CH / kWave;
  const int ni = (nins + G - 1) / G;
  auto dma = [&](const uint16_t* src_rows, uint16_t* dst) {   // rows t0.. of a tile
    const uint64_t src = (uint64_t)(uintptr_t)src_rows;
    const uint32_t slo = __builtin_amdgcn_readfirstlane((uint32_t)src);
    const uint32_t shi = __builtin_amdgcn_readfirstlane((uint32_t)(src >> 32));
    const uint64_t sbase = ((uint64_t)shi << 32) | slo;
    for (int x = 0; x < ni; ++x) {
      int ins = wave + G * x;
      ins = ins < nins ? ins : nins - 1;
      const int chunk = ins * kWave + lane, r = chunk / CH, cc = chunk % CH;
      const uint32_t voff = (uint32_t)((r * rs + 8 * cc) * 2);
      const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(lds_void*)((char*)dst + ins * 1024));
      uint32_t m0_saved;
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(m0_saved)
          : "s"(lds0), "v"(voff), "s"(sbase)
          : "memory", "scc");
    }
  };
  // the split's entries that name a block of the cache, in order
  auto next_valid = [&](int e) -> int {       // (scalar loads: a vector load here would wait
    for (; e < e1; ++e) {                     // for the transfers in flight)
      const int j = row[__builtin_amdgcn_readfirstlane(e)];
      if (j >= 0 && (int64_t)j * block < L) break;   // else an unused place or beyond the cache
    }
    return e;
  };
  __syncthreads();
  float qv[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) qv[x] = qsm[wave * D + 8 * dg + x];
  int e = len_ok ? next_valid(e0) : e1;
  if (e < e1) {
    const int64_t t0 = (int64_t)row[e] * block;
    dma(kb0 + t0 * rs, Ks);
    dma(vb0 + t0 * rs, Vs);
  }
  while (e < e1) {
    const int en = next_valid(e + 1);
    const int64_t t0 = (int64_t)row[e] * block;
    const int nk = (int)(L - t0 < block ? L - t0 : block);   // own block: tokens < L
    dwait_vmcnt_le(ni);                       // this wave's keys of block e (values may fly)
    __syncthreads();                          // every wave's keys landed
    for (int t = kq; t < nk; t += KG) {
      const u32x4 kw = *(const u32x4*)(Ks + t * D + 8 * dg);
      float a = 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        a = __builtin_fmaf(qv[2 * x], bf16lo(kw[x]), a);
        a = __builtin_fmaf(qv[2 * x + 1], bf16hi(kw[x]), a);
      }
      a = group_sum<LG>(a);
      if (dg == 0) psm[wave * block + t] = a * c;       // exp2 domain
    }
    __syncthreads();                          // scores written; every wave done with Ks
    if (en < e1) dma(kb0 + (int64_t)row[en] * block * rs, Ks);
    float s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = lane + 64 * u;
      s[u] = t < nk ? psm[wave * block + t] : -__builtin_inff();
    }
    float mb = fmaxf(s[0], s[1]);
    mb = wave_max(mb);
    const float mn = fmaxf(m, mb);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);    // 0 on the first block
    m = mn;
    float lp = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {             // (each wave reads and writes its own row)
      const int t = lane + 64 * u;
      const float p = t < nk ? __builtin_amdgcn_exp2f(s[u] - m) : 0.f;
      if (t < block) psm[wave * block + t] = p;
      lp += p;
    }
    lp = wave_sum(lp);
    l = l * alpha + lp;
#pragma unroll
    for (int x = 0; x < 8; ++x) o[x] *= alpha;
    if (en < e1) dwait_vmcnt_le(ni); else dwait_vmcnt<0>();   // values of block e
    __syncthreads();                          // every wave's values landed, weights written
    for (int t = kq; t < nk; t += KG) {
      const u32x4 vw = *(const u32x4*)(Vs + t * D + 8 * dg);
      const float p = psm[wave * block + t];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        o[2 * x] = __builtin_fmaf(p, bf16lo(vw[x]), o[2 * x]);
        o[2 * x + 1] = __builtin_fmaf(p, bf16hi(vw[x]), o[2 * x + 1]);
      }
    }
    __syncthreads();                          // every wave done with Vs and its weights
    if (en < e1) dma(vb0 + (int64_t)row[en] * block * rs, Vs);
    e = en;
  }
  // sum the key groups (lanes dg, dg + LG, ...)
#pragma unroll
  for (int off = LG; off < 64; off <<= 1)
#pragma unroll
    for (int x = 0; x < 8; ++x) o[x] += __shfl_xor(o[x], off);
  if (kq == 0) {
#pragma unroll
    for (int x = 0; x < 8; ++x) my[2 + 8 * dg + x] = o[x];
  }
  if (lane == 0) {
    my[0] = m;
    my[1] = l;
  }
}

template <int D>
__global__ __launch_bounds__(64) void dcombine_kernel(const float* __restrict__ part,
                                                      const int32_t* __restrict__ lens,
                                                      uint16_t* __restrict__ out, int64_t Lmax,
                                                      int Hq, int splits) {
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const float* pp = part + (int64_t)bh * splits * (D + 2);
  float M = -__builtin_inff();
  for (int s = 0; s < splits; ++s) M = fmaxf(M, pp[s * (D + 2)]);
  float lsum = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float ms = pp[s * (D + 2)];
    if (ms != -__builtin_inff()) lsum += __builtin_amdgcn_exp2f(ms - M) * pp[s * (D + 2) + 1];
  }
  const int64_t L = lens[b];
  const bool ok = L >= 1 && L <= Lmax && lsum > 0.f;
  for (int d = threadIdx.x; d < D; d += 64) {
    float acc = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float ms = pp[s * (D + 2)];
      if (ms != -__builtin_inff()) acc += __builtin_amdgcn_exp2f(ms - M) * pp[s * (D + 2) + 2 + d];
    }
    const float v = ok ? acc / lsum : __builtin_nanf("");
    out[(int64_t)bh * D + d] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
  }
}

template <int D, int CPL>
hipError_t launch_dsel(const void* q, const float* kbar, const int32_t* lens, int32_t* idx,
                       int64_t Lmax, int Hq, int Hkv, int block, int nbmax, int topk,
                       unsigned heads, bool group, hipStream_t stream) {
  if constexpr (CPL <= 32)                    // nb <= 2048: 4 waves per (sequence, head)
    dselect_kernel<D, CPL, 4><<<heads, 256, 0, stream>>>(
        (const uint16_t*)q, kbar, lens, idx, Lmax, Hq, Hkv, block, nbmax, topk, (int)heads, group);
  else
    dselect_kernel<D, CPL, 1><<<(heads + kSelWaves - 1) / kSelWaves, kSelWaves * 64, 0, stream>>>(
        (const uint16_t*)q, kbar, lens, idx, Lmax, Hq, Hkv, block, nbmax, topk, (int)heads, group);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dselect(const void* q, const float* kbar, const int32_t* lens, int32_t* idx,
                          int64_t Lmax, int Hq, int Hkv, int block, int nbmax, int topk,
                          unsigned heads, bool group, hipStream_t stream) {
  if (nbmax <= 64) return launch_dsel<D, 1>(q, kbar, lens, idx, Lmax, Hq, Hkv, block, nbmax, topk, heads, group, stream);
  if (nbmax <= 256) return launch_dsel<D, 4>(q, kbar, lens, idx, Lmax, Hq, Hkv, block, nbmax, topk, heads, group, stream);
  if (nbmax <= 1024) return launch_dsel<D, 16>(q, kbar, lens, idx, Lmax, Hq, Hkv, block, nbmax, topk, heads, group, stream);
  if (nbmax <= 2048) return launch_dsel<D, 32>(q, kbar, lens, idx, Lmax, Hq, Hkv, block, nbmax, topk, heads, group, stream);
  if (nbmax <= 4096) return launch_dsel<D, 64>(q, kbar, lens, idx, Lmax, Hq, Hkv, block, nbmax, topk, heads, group, stream);
  return launch_dsel<D, kSelCols>(q, kbar, lens, idx, Lmax, Hq, Hkv, block, nbmax, topk, heads, group, stream);
}

}  // namespace

// The most splits a decode step uses (the workspace is sized for it): up to 8192 waves of the
// per-head kernel, at most 64, at most topk. The launch picks fewer (launch_splits below).
int decode_splits(int64_t B, int Hq, int topk) {
  const int64_t heads = B * Hq;
  int64_t s = (8192 + heads - 1) / heads;
  if (s > topk) s = topk;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

namespace {

// Splits of each head's (or KV head's) selected blocks for the attention pass. Every wave's
// blocks are a chain of dependent tile loads, and the step is bound by HBM: about 16 waves
// per CU in flight saturate the reads, and a second round of work-groups adds a whole chain
// of latency, so the launch aims at 16 waves per CU and never at more work-groups than the
// chip holds at once (occupancy query). Measured on 32 sequences x 32768 cached tokens,
// 32/8 heads, 76 blocks: per-head kernel 2, 3, 4, 5, 6, 8 splits 0.561, 0.466, 0.444, 0.455,
// 0.539, 0.476 ms; group kernel (4 waves per work-group, 4 resident per CU) 3, 4, 5, 8 splits
// 0.188, 0.174, 0.205, 0.182 ms: both best at 16 waves per CU.
hipError_t launch_splits(int64_t units, int waves_per_unit, const void* fn, int threads,
                         size_t lds, int max_splits, int* splits) {
  int dev = 0, ncu = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds);
  if (e != hipSuccess) return e;
  if (units < 1) units = 1;
  int64_t s = (int64_t)16 * ncu / (units * waves_per_unit);          // 16 waves per CU
  const int64_t fill = (int64_t)ncu * (per_cu > 0 ? per_cu : 1) / units;   // one round
  if (s > fill) s = fill;
  if (s > max_splits) s = max_splits;
  if (s < 1) s = 1;
  *splits = (int)s;
  return hipSuccess;
}

}  // namespace

size_t decode_workspace_bytes(int64_t B, int Hq, int D, int topk) {
  return (size_t)B * Hq * decode_splits(B, Hq, topk) * (D + 2) * sizeof(float);
}

bool decode_supported(int D, int block) {
  return (D == 64 || D == 128) && (block == 64 || block == 128);
}

hipError_t launch_decode_pool(int64_t B, int64_t Lmax, int Hkv, int D, int block,
                              const void* k_cache, const int32_t* lens_old,
                              const int32_t* lens_new, float* kbar, hipStream_t stream) {
  const int nbmax = (int)(Lmax / block);
  pool_new_kernel<<<dim3((unsigned)nbmax, (unsigned)B), 256, 0, stream>>>(
      (const uint16_t*)k_cache, lens_old, lens_new, kbar, Lmax, Hkv, D, block, nbmax);
  return hipGetLastError();
}

hipError_t launch_decode(int64_t B, int64_t Lmax, int Hq, int Hkv, int D, int block, int topk,
                         bool group, const void* q, const void* k_cache, const void* v_cache,
                         const float* kbar, const int32_t* lens, float scale, void* out,
                         int32_t* idx, void* workspace, hipStream_t stream) {
  const int nbmax = (int)(Lmax / block);
  int splits = decode_splits(B, Hq, topk);
  const float c = (float)((double)scale * 1.4426950408889634);
  float* part = (float*)workspace;
  const unsigned heads = (unsigned)(B * Hq);
  const unsigned sel_rows = (unsigned)(B * (group ? Hkv : Hq));   // selection rows
  hipError_t e = D == 64 ? launch_dselect<64>(q, kbar, lens, idx, Lmax, Hq, Hkv, block, nbmax,
                                              topk, sel_rows, group, stream)
                         : launch_dselect<128>(q, kbar, lens, idx, Lmax, Hq, Hkv, block, nbmax,
                                               topk, sel_rows, group, stream);
  if (e != hipSuccess) return e;
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = Hq / Hkv;
  if (group && G > 1 && G <= kMaxDecodeGroup) {   // one work-group per (b, KV head, split)
    const size_t lds = (size_t)2 * block * D * 2 + (size_t)G * (D + block) * sizeof(float);
    const void* fn = D == 64 ? reinterpret_cast<const void*>(&dattn_group_kernel<64>)
                             : reinterpret_cast<const void*>(&dattn_group_kernel<128>);
    if (lds > 65536) {                        // beyond the default dynamic LDS of a launch
      const hipError_t ea =
          hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (ea != hipSuccess) return ea;
    }
    e = launch_splits(B * Hkv, G, fn, G * 64, lds, splits, &splits);
    if (e != hipSuccess) return e;
    const unsigned groups = (unsigned)(B * Hkv * splits);
    if (D == 64)
      dattn_group_kernel<64><<<groups, G * 64, lds, stream>>>(
          (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache, idx, lens,
          part, Lmax, Hq, Hkv, block, topk, splits, c);
    else
      dattn_group_kernel<128><<<groups, G * 64, lds, stream>>>(
          (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache, idx, lens,
          part, Lmax, Hq, Hkv, block, topk, splits, c);
  } else {
    const void* fn = D == 64 ? reinterpret_cast<const void*>(&dattn_kernel<64>)
                             : reinterpret_cast<const void*>(&dattn_kernel<128>);
    e = launch_splits(B * Hq, 1, fn, 64, 0, splits, &splits);
    if (e != hipSuccess) return e;
    if (D == 64)
      dattn_kernel<64><<<heads * splits, 64, 0, stream>>>(
          (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache, idx, lens,
          part, Lmax, Hq, Hkv, block, topk, splits, c);
    else
      dattn_kernel<128><<<heads * splits, 64, 0, stream>>>(
          (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache, idx, lens,
          part, Lmax, Hq, Hkv, block, topk, splits, c);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (D == 64)
    dcombine_kernel<64><<<heads, 64, 0, stream>>>(part, lens, (uint16_t*)out, Lmax, Hq, splits);
  else
    dcombine_kernel<128><<<heads, 64, 0, stream>>>(part, lens, (uint16_t*)out, Lmax, Hq, splits);
  return hipGetLastError();
}

}  // namespace bsattn
