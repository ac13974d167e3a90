// Step 4: attention over the gathered selected blocks, bf16 inputs, bf16 MFMA (gfx950).
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"), section
// "SparseFormer 注意力实现", step 3: attention is computed only over the selected blocks with
// scale 1/sqrt(D); MSA page ("从M2.7到M3：多模态模型稀疏注意力架构设计与实现全解析") §2.1:
// Softmax(Mask(Q K^T / sqrt(d_k))) V with a block mask, §2.2: full attention inside the chosen
// blocks, §3.1: GQA. The softmax is exact: it is evaluated online over the k selected key
// blocks with a reference maximum and a normaliser in fp32.
//
// Work split: one work-group owns the query rows of one query block of one (batch, query
// head); each of its waves owns QW query rows (QW = 64 for D = 64, 32 for D = 128), i.e. QW/32
// column tiles of the 32x32 MFMA. A 128-token selected block is walked in two 64-key steps,
// so that one step's operands fit in registers with two waves per SIMD while every gathered
// tile is still fetched once per query block. Per step each wave computes
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q^T in registers)
//   P^T = exp2(c*S^T - m)   (c = scale*log2(e), m = row reference, usually 0)
//   O^T += V^T P^T (A = V^T via ds_read_b64_tr_b16 transpose reads of the row-major V tile,
//                   B = P^T built straight from the S^T accumulators)
// Each A operand read from LDS feeds all QW/32 column tiles of the wave.
// Working on the transposed products keeps each query's key scores in two lanes (l, l^32),
// and the score accumulators are already in the B-operand layout of the next product: the 16
// k-slots of a step are matched to keys {4h..4h+3, 8+4h..8+4h+3} on both operands.
//
// Data movement: K and V tiles go from HBM/L2 straight into LDS with global_load_lds_dwordx4
// (lane l of one instruction fills bytes [16l, 16l+16) of a 1 KiB LDS span; the lane fetches
// whichever 16-byte chunk belongs there). One wave per work-group (D = 64, 64-token blocks):
// one LDS buffer per tensor; the wave reads all K operands of step t into registers, then
// starts the K transfer of step t+1 and computes S^T and the softmax while it flies; V likewise
// before the PV product (with several waves and 16 KiB tiles the same, with barriers around the
// reads). Otherwise, several waves per work-group: two buffers per tensor; after one barrier at
// the start of step t (every wave's share of step t landed, every wave done with step t-1) the
// K and V tiles of step t+1 start into the other buffers.
// LDS bank layout: gfx950's LDS has 64 banks of 4 bytes (256 bytes per clock); a 16-byte row
// read serves 16 lanes per clock and an 8-byte transpose read 32 lanes. The 16-byte chunk c of
// tile row r sits at chunk position c ^ f(r), with f chosen so that every such group of lanes
// covers the 64 banks once: at D = 64 (128-byte rows, two per bank line) f(r) = 4((r>>1)&1) +
// ((r>>2)&3), which gives the 8 even and the 8 odd rows of a 16-row K read 8 distinct chunk
// positions each and puts rows r and r+2 of a V transpose read on opposite halves of the row;
// at D = 128 (256-byte rows, one per bank line) f(r) = 4(r&3) + ((r>>2)&3) over 16 chunks,
// which gives 16 consecutive rows 16 distinct positions and each 4-row group of a V transpose
// read its own quarter of the row.
//
// Softmax reference: softmax does not depend on the reference value m subtracted from a row
// (p = exp2(c*s - m), c = scale*log2(e)), so m stays 0 while every per-lane step sum of
// weights lies in [2^-64, 2^64], which holds for inputs of moderate range: no row max and no
// rescale are needed. The row is first done with m = 0 throughout, only noting whether a step
// left that range; a flagged row (huge or tiny scores) is done again from the start, and that
// pass moves the reference to the running max whenever a step leaves the range, rescaling O
// and l by exp2(m_old - m_new). O and l always share one reference. A row whose output sums
// are not finite after that (values near the top of the bf16 range times weights up to 2^64)
// is done once more with the upper bound of the range lowered to 1: the reference then
// follows the running maximum and every weight is at most 1, as in a max-referenced softmax. The normaliser sums the
// fp32 weights with plain adds (measured: the bf16 dot instruction waits for MFMAs in flight,
// so it cannot hide under them); the PV product takes the same weights rounded to bf16.
//
// Causal variant (template flag): query block i reads the first min(topk, i+1) entries of its
// row, each of which must lie in [0, i]; in its own block i the scores of keys after the
// query are set to -inf before the weights (weight 0).
//
// Overlapping key blocks (template flag; the MSA page's §5.3 overlap remedy): the row's key
// blocks are marked in an LDS bitmap, block j is read from its tile at key_tile_start and
// the tile's first key_tile_skip keys score -inf, so the union of the row's blocks counts
// each token once.
#pragma once

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

constexpr float kSumHi = 18446744073709551616.0f;          // 2^64
constexpr float kSumLo = 1.0f / 18446744073709551616.0f;   // 2^-64

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const char lds_char;
typedef __attribute__((address_space(1))) const void global_cvoid;

// R query rows per work-group, KU keys per step (one K and one V tile in LDS)
template <int D, int R, int KU>
struct Cfg {
  static constexpr int QW = D == 64 ? 64 : 32;  // query rows per wave
  static constexpr int QC = QW / 32;           // 32-query column tiles per wave
  static constexpr int NW = R / QW;            // waves
  static constexpr int NT = NW * kWave;        // threads
  static constexpr int TILE = KU * D * 2;      // bytes of one K or V tile
  static constexpr int DMA = TILE / 1024 / NW; // 1 KiB transfers per tile per wave
  static constexpr int NKT = KU / 32;          // 32-key sub-tiles per step
  static constexpr int NS = D / 16;            // k-steps of Q K^T
  static constexpr int NDT = D / 32;           // 32-row d tiles of O^T
  static constexpr int NPS = KU / 16;          // k-steps of V^T P^T
  static_assert(DMA * NW * 1024 == TILE, "tile must split into whole 1 KiB transfers");
  static_assert(DMA == 4 || DMA == 8, "the transfer sequences issue 4 or 8 spans of 1 KiB");
};

// vmcnt-only waits (expcnt and lgkmcnt left free), gfx9 s_waitcnt encoding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// chunk position of logical 16-byte chunk c in tile row r (an involution in c)
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 64) return c ^ (4 * ((r >> 1) & 1) + ((r >> 2) & 3));
  else return c ^ (4 * (r & 3) + ((r >> 2) & 3));
}

__device__ __forceinline__ s16x4 ds_read_tr16(const lds_char* lds_bytes) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_bytes));
}

// A work-group takes R rows of a query block of SB tokens (R = SB, or R = 64: SB / R
// work-groups per query block) and walks each selected block in steps of KU keys (SB / KU
// steps). KU = 64 keeps one step's operands in registers with two waves per SIMD; a whole
// 128-key step needs them all at once (one wave per SIMD). R = SB reads each gathered tile
// once per query block, R = 64 once per row part.
//
// OVL: overlapping key blocks (key block j starts at token j*kstride; nkb of them): the tile of
// block j starts at key_tile_start and its first key_tile_skip keys score -inf.
template <int D, int SB, int R, int KU, bool CAUSAL, bool OVL>
__global__ __launch_bounds__(R / (D == 64 ? 64 : 32) * 64) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, uint16_t* __restrict__ out,
    float* __restrict__ lse, int64_t N, int Hq, int Hkv, int nb, int topk, float c,
    uint32_t total_tiles, int nkb, int kstride) {
  constexpr int RP = SB / R;                  // work-groups (row parts) per query block
  constexpr int UN = SB / KU;                 // steps per selected block
  using C = Cfg<D, R, KU>;
  // With one wave per work-group each tensor has one LDS buffer (its transfers are waited for
  // by that wave alone). With several waves sharing the tiles, two buffers per tensor: the
  // tiles of step t+1 go into the other buffer at the start of step t, after one barrier that
  // also ends every wave's reads of step t-1 (one barrier per step, not four).
  // (Two waves with 16 KiB tiles keep one buffer: 64 KiB per work-group would leave one wave
  // per SIMD.)
  constexpr int NBUF = (C::NW >= 4 || (C::NW == 2 && C::TILE <= 8192)) ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) char Kl[NBUF][C::TILE];   // [KU][D] bf16, swizzled
  __shared__ __attribute__((aligned(1024))) char Vl[NBUF][C::TILE];
  __shared__ uint32_t chosen[OVL ? kMaxKeyBlocks / 32 : 1];   // OVL: the row's key blocks

  // tile order: (b, kv head, query block, head within group, row part); blocks reading the
  // same K/V are consecutive and land on one XCD, and the G heads of a query block (which
  // read the same tiles under a group-shared selection) run side by side
  const uint32_t tile = xcd_remap(blockIdx.x, total_tiles);
  const int G = Hq / Hkv;
  const int hq = (int)(tile % RP);            // which R rows of the query block
  uint32_t rest = tile / RP;
  const int hh = (int)(rest % G);
  rest /= G;
  const int i = (int)(rest % nb);
  rest /= nb;
  const int g = (int)(rest % Hkv);
  const int b = (int)(rest / Hkv);
  const int h = g * G + hh;

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t qrs = (int64_t)Hq * D;         // token stride of q/out
  const int64_t krs = (int64_t)Hkv * D;        // token stride of k/v

  // Q^T as B operands: lane holds q[row = QW*wave + 32*qc + l32][d = 16s + 8*half .. +7]
  const int64_t qrow0 = (int64_t)b * N + (int64_t)i * SB + R * hq + C::QW * wave + l32;
  bf16x8 qf[C::QC][C::NS];
#pragma unroll
  for (int qc = 0; qc < C::QC; ++qc)
#pragma unroll
    for (int s = 0; s < C::NS; ++s)
      qf[qc][s] = __builtin_bit_cast(
          bf16x8, *(const u32x4*)(q + (qrow0 + 32 * qc) * qrs + (int64_t)h * D + 16 * s + 8 * half));

  const int32_t* myidx = idx + (((int64_t)b * Hq + h) * nb + i) * topk;
  const char* kbase0 = (const char*)(k + (int64_t)b * N * krs + (int64_t)g * D);
  const char* vbase0 = (const char*)(v + (int64_t)b * N * krs + (int64_t)g * D);
  const int kcount = CAUSAL && i + 1 < topk ? i + 1 : topk;   // entries of the row used
  const unsigned klim = CAUSAL ? (unsigned)(i + 1) : (unsigned)(OVL ? nkb : nb);   // admissible

  // DMA source byte offsets of this lane inside a tile (fixed), destination spans uniform
  uint32_t goff[C::DMA];
#pragma unroll
  for (int x = 0; x < C::DMA; ++x) {
    const int pos = (wave * C::DMA + x) * 64 + lane;         // chunk position in the tile
    const int r = pos / (D / 8), p = pos % (D / 8);
    goff[x] = (uint32_t)((r * krs + swz<D>(r, p) * 8) * 2);
  }
  bool bad = false;
  auto tile_base = [&](int kb, int u) -> int64_t {   // step u (KU keys) of selected block kb
    if ((unsigned)kb >= klim) { bad = true; kb = 0; }
    const int64_t first = OVL ? key_tile_start(kb, kstride, SB, N) : (int64_t)kb * SB;
    return (first + KU * u) * krs * 2;
  };
  auto skip_of = [&](int kb) -> int {          // OVL: leading keys of kb's tile left out
    if (!OVL || (unsigned)kb >= klim) return 0;
    return key_tile_skip(kb, kstride, SB, N, is_selected(chosen, kb - 1));
  };
  // The transfers are issued from inline asm so that the compiler's wait-count pass, which
  // cannot tell the K and V buffers apart, does not add full vmcnt(0) waits before every LDS
  // read; the waits below are placed by hand (each wave issues exactly DMA transfers per tile
  // and no other vector-memory instruction inside the loop). M0 (the LDS destination) is
  // saved and restored around them.
  // LDS byte addresses of the tile buffers, taken once from the arrays themselves (the loop
  // works with these and with LDS-typed pointers only, no generic-pointer casts)
  const uint32_t kl_addr = (uint32_t)(uintptr_t)(lds_void*)&Kl[0][0];
  const uint32_t vl_addr = (uint32_t)(uintptr_t)(lds_void*)&Vl[0][0];
  auto dma = [&](const char* src_base_any, uint32_t dst_lds) {
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(dst_lds + wave * C::DMA * 1024);
    // the source base is the same in every lane; readfirstlane keeps it in scalar registers
    // where the compiler cannot prove that (the asm operand below must be an SGPR pair)
    const uint64_t sb = (uint64_t)(uintptr_t)src_base_any;
    const char* src_base = (const char*)(uintptr_t)(
        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sb) |
        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sb >> 32)) << 32));
    uint32_t m0_saved;
    if constexpr (C::DMA == 4) {
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %6\n\t"
          "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %6\n\t"
          "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %6\n\t"
          "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, %6\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(m0_saved)
          : "s"(lds0), "v"(goff[0]), "v"(goff[1]), "v"(goff[2]), "v"(goff[3]), "s"(src_base)
          : "memory", "scc");
      return;
    } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %10\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %10\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %10\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, %10\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, %10\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %7, %10\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %8, %10\n\t"
        "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %9, %10\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0_saved)
        : "s"(lds0), "v"(goff[0]), "v"(goff[1]), "v"(goff[2]), "v"(goff[3]), "v"(goff[4]),
          "v"(goff[5]), "v"(goff[6]), "v"(goff[7]), "s"(src_base)
        : "memory", "scc");
    }
  };

  // LDS read offsets of this lane
  int koff[C::NS];                             // K row l32, chunk 2s+half (+ 32*kt rows)
#pragma unroll
  for (int s = 0; s < C::NS; ++s) koff[s] = l32 * D * 2 + 16 * swz<D>(l32, 2 * s + half);
  // V transpose reads: in each 16-lane group lane 4e+t names row 4*half+e (+16s, +8) and
  // columns 32dt + 16*((lane>>4)&1) + 4t, i.e. chunk 4dt + 2*((lane>>4)&1) + t/2, half t&1
  // (rows r and r + 8 have their own chunk positions: f depends on bit 3 of the row)
  int voff[C::NDT], voff8[C::NDT];
  {
    const int e = (lane & 15) >> 2, r = 4 * half + e;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      const int ch = 4 * dt + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
      voff[dt] = r * D * 2 + 16 * swz<D>(r, ch) + 8 * (lane & 1);
      voff8[dt] = (r + 8) * D * 2 + 16 * swz<D>(r + 8, ch) + 8 * (lane & 1);
    }
  }

  f32x16 oacc[C::NDT][C::QC];
  float mc[C::QC], lsum[C::QC];               // reference (exp2 domain); lane's normaliser share

  if (OVL) mark_selected(chosen, myidx, kcount, nkb, tid, C::NT);
  // Q must have landed before the first transfer: the hand-placed vmcnt waits in the loop
  // count transfers only (the empty asm consumes the loaded registers here)
#pragma unroll
  for (int qc = 0; qc < C::QC; ++qc)
#pragma unroll
    for (int s = 0; s < C::NS; ++s) asm volatile("" ::"v"(qf[qc][s]));

  // One pass over the row's steps. The first pass (CHECKED = false) keeps the reference at 0
  // and only records whether some step's weight sum left [2^-64, 2^64]; rows it flags are
  // done again from the start with CHECKED = true, which moves the reference to the row max
  // whenever that happens. Taking the check out of the common pass lets the weights, the
  // normaliser and the products of consecutive steps overlap.
  auto pass = [&](auto checked_tag, float sum_hi) -> bool {
    constexpr bool CHECKED = decltype(checked_tag)::value;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int qc = 0; qc < C::QC; ++qc)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][qc][r] = 0.f;
#pragma unroll
    for (int qc = 0; qc < C::QC; ++qc) { mc[qc] = 0.f; lsum[qc] = 0.f; }
    bool flagged = false;
    int kb_cur = myidx[0], u_cur = 0;
    int skip_cur = skip_of(kb_cur);
    {
      const int64_t tb = tile_base(kb_cur, 0);
      dma(kbase0 + tb, kl_addr);
      dma(vbase0 + tb, vl_addr);
    }

    // one step; with two buffers their index is a compile-time constant (the loop below takes
    // steps two at a time), so the LDS read addresses stay fixed and the buffer goes into the
    // offset field
    auto step = [&](int t, auto buf) {
      const bool more = t + 1 < kcount * UN;
      const int kb_next = more ? myidx[(t + 1) / UN] : 0;
      const int u_next = (t + 1) % UN;
      const int64_t tb_next = more ? tile_base(kb_next, u_next) : 0;
      const int skip_next = OVL && more ? skip_of(kb_next) : 0;

      // ---- K(t): wait for this wave's share (V(t) may still fly), then the whole work-group
      int cur = 0;                              // run-time index: D = 64 with two buffers
      if constexpr (std::is_same_v<decltype(buf), int>) cur = NBUF > 1 ? (t & 1) : 0;
      else cur = decltype(buf)::value;
      const char* Kc = Kl[cur];
      lds_char* Vc = (lds_char*)(uintptr_t)(vl_addr + cur * C::TILE);
      if constexpr (NBUF > 1) {
        wait_vmcnt<0>();                       // this wave's share of step t's tiles
        __syncthreads();                       // every share landed; step t-1 read everywhere
        if (more) {
          dma(kbase0 + tb_next, kl_addr + (cur ^ 1) * C::TILE);
          dma(vbase0 + tb_next, vl_addr + (cur ^ 1) * C::TILE);
        }
      } else {
        wait_vmcnt<C::DMA>();                  // K(t) (V(t) may still fly)
        if (C::NW > 1) __syncthreads();
      }
      bf16x8 ka[C::NKT][C::NS];
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int s = 0; s < C::NS; ++s)
          ka[kt][s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(Kc + kt * 32 * D * 2 + koff[s]));
      if constexpr (NBUF == 1) {
        wait_lgkmcnt0();
        if (C::NW > 1) __syncthreads();        // every wave's K(t) reads done
        if (more) dma(kbase0 + tb_next, kl_addr);
      }

      // ---- S^T = K Q^T
      f32x16 sacc[C::NKT][C::QC];
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int qc = 0; qc < C::QC; ++qc) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kt][qc][r] = 0.f;
#pragma unroll
          for (int s = 0; s < C::NS; ++s)
            sacc[kt][qc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kt][s], qf[qc][s], sacc[kt][qc], 0, 0, 0);
        }
      if (CAUSAL && kb_cur == i) {               // own block: keys after the query get -inf
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
          for (int qc = 0; qc < C::QC; ++qc)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = KU * u_cur + 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
              const int qry = R * hq + C::QW * wave + 32 * qc + l32;
              if (key > qry) sacc[kt][qc][r] = -__builtin_inff();
            }
      }
      if (OVL && skip_cur > KU * u_cur) {        // keys before the block or held by block kb-1
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
          for (int qc = 0; qc < C::QC; ++qc)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = KU * u_cur + 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
              if (key < skip_cur) sacc[kt][qc][r] = -__builtin_inff();
            }
      }

      // At D = 64 the weights' VALU work equals the MFMA work; issuing it at a raised wave
      // priority (back to normal for the PV product) keeps it flowing while the other wave on
      // the SIMD multiplies (measured: 2.91 -> 2.83 ms on the page's shape; slower at D = 128)
      if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
      // ---- softmax weights (lane pair l, l^32 shares one query row): p = exp2(c*s - m), m the
      // row reference in the exp2 domain (0 until a block sum leaves [2^-64, 2^64])
      auto row_max = [&](int qc) {
        float mt = sacc[0][qc][0];
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kt][qc][r]);
        return fmaxf(mt, __shfl_xor(mt, 32)) * c;
      };
      uint32_t pw[C::QC][C::NPS][4];
      float bsum[C::QC];
      auto weights = [&](int qc) {
        float sa = -0.f, sb = -0.f;              // two add chains (x + -0 folds to x)
#pragma unroll
        for (int s = 0; s < C::NPS; ++s)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(
                __builtin_fmaf(sacc[s >> 1][qc][8 * (s & 1) + 2 * e], c, -mc[qc]));
            const float p1 = __builtin_amdgcn_exp2f(
                __builtin_fmaf(sacc[s >> 1][qc][8 * (s & 1) + 2 * e + 1], c, -mc[qc]));
            const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
            pw[qc][s][e] = __builtin_bit_cast(uint32_t, pp);
            sa += p0;
            sb += p1;
          }
        bsum[qc] = sa + sb;
      };
#pragma unroll
      for (int qc = 0; qc < C::QC; ++qc) weights(qc);
      bool off_range = false;
#pragma unroll
      for (int qc = 0; qc < C::QC; ++qc)
        off_range |= (bsum[qc] > sum_hi) || (lsum[qc] + bsum[qc] < kSumLo);
      if (!CHECKED) flagged |= off_range;
      if (CHECKED && __ballot(off_range)) {      // move the reference to the row max
#pragma unroll
        for (int qc = 0; qc < C::QC; ++qc) {
          const float bm = row_max(qc);
          const float l_row = lsum[qc] + __shfl_xor(lsum[qc], 32);   // same on both lanes
          if (l_row == 0.f) {                    // nothing accumulated yet: O and l are zero
            if (bm != -__builtin_inff()) mc[qc] = bm;   // (a step whose keys are all left out)
          } else {
            const float m_new = fmaxf(mc[qc], bm);
            const float alpha = __builtin_amdgcn_exp2f(mc[qc] - m_new);
            lsum[qc] *= alpha;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[dt][qc][r] *= alpha;
            mc[qc] = m_new;
          }
          weights(qc);
        }
      }
#pragma unroll
      for (int qc = 0; qc < C::QC; ++qc) lsum[qc] += bsum[qc];

      // ---- V(t): (one buffer: wait, K(t+1) may still fly) read all V^T operands, then start
      // V(t+1)
      if constexpr (NBUF == 1) {
        if (more) wait_vmcnt<C::DMA>(); else wait_vmcnt<0>();
        if (C::NW > 1) __syncthreads();
      }
      bf16x8 va[C::NPS][C::NDT];
#pragma unroll
      for (int s = 0; s < C::NPS; ++s)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
          lds_char* p = Vc + (16 * s) * D * 2;
          const s16x4 a8[2] = {ds_read_tr16(p + voff[dt]), ds_read_tr16(p + voff8[dt])};
          va[s][dt] = __builtin_bit_cast(bf16x8, a8);
        }
      if constexpr (NBUF == 1) {
        wait_lgkmcnt0();                       // V(t) read before V(t+1) overwrites it
        if (C::NW > 1) __syncthreads();
        if (more) dma(vbase0 + tb_next, vl_addr);
      }

      // ---- O^T += V^T P^T
      if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int s = 0; s < C::NPS; ++s)
#pragma unroll
        for (int qc = 0; qc < C::QC; ++qc) {
          const u32x4 pv = {pw[qc][s][0], pw[qc][s][1], pw[qc][s][2], pw[qc][s][3]};
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pv);
#pragma unroll
          for (int dt = 0; dt < C::NDT; ++dt)
            oacc[dt][qc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[s][dt], pb, oacc[dt][qc], 0, 0, 0);
        }
      kb_cur = kb_next;
      u_cur = u_next;
      if (OVL) skip_cur = skip_next;
    };
    if constexpr (NBUF > 1 && D == 128 && !OVL) {   // (with OVL it would need > 256 registers)
      for (int t = 0; t < kcount * UN; t += 2) {
        step(t, std::integral_constant<int, 0>{});
        if (t + 1 < kcount * UN) step(t + 1, std::integral_constant<int, 1>{});
      }
    } else {
      for (int t = 0; t < kcount * UN; ++t) step(t, -1);
    }
    return flagged;
  };
  // whether this lane's output sums are all finite (the reference 0 lets weights reach 2^64
  // per step, so values near the top of the bf16 range can overflow where a max-referenced
  // softmax would not)
  auto finite = [&]() -> bool {
    bool fin = true;
#pragma unroll
    for (int qc = 0; qc < C::QC; ++qc) {
      fin &= __builtin_isfinite(lsum[qc]);
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) fin &= __builtin_isfinite(oacc[dt][qc][r]);
    }
    return fin;
  };
  // the decision is work-group-wide: the waves of a work-group share the tiles and barriers.
  // The causal and overlapping-block variants keep a single checked pass (their extra masking
  // leaves no registers for a second copy of the loop with two waves per SIMD).
  // A row whose sums are not finite after that is done once more with the upper bound 1:
  // its reference then follows the running row maximum and no weight exceeds 1.
  // (one inlined copy of each pass: the checked pass runs in a loop; the decisions are
  // work-group-wide, made wave-uniform for the compiler with readfirstlane)
  auto all_or = [](bool x) -> bool {
    return __builtin_amdgcn_readfirstlane(__syncthreads_or(x) ? 1 : 0) != 0;
  };
  float hi = kSumHi;
  bool again = true;
  if constexpr (!(CAUSAL || OVL)) {
    again = all_or(pass(std::false_type{}, kSumHi));
    if (!again && all_or(!finite())) { again = true; hi = 1.0f; }
  }
  while (again) {
    pass(std::true_type{}, hi);
    again = hi != 1.0f && all_or(!finite());
    hi = 1.0f;
  }

  // epilogue: O = O^T / l, bf16, 4 consecutive d per store
#pragma unroll
  for (int qc = 0; qc < C::QC; ++qc) {
    const float l_all = lsum[qc] + __shfl_xor(lsum[qc], 32);
    const float inv = bad ? __builtin_nanf("") : 1.0f / l_all;
    uint16_t* orow = out + (qrow0 + 32 * qc) * qrs + (int64_t)h * D;
    if (lse && half == 0)                      // natural log-sum-exp of the row's scaled scores
      lse[((int64_t)b * Hq + h) * N + (qrow0 - (int64_t)b * N) + 32 * qc] =
          bad ? __builtin_nanf("") : (mc[qc] + log2f(l_all)) * 0.6931471805599453f;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * dt + 8 * j + 4 * half;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[dt][qc][4 * j + 0] * inv, oacc[dt][qc][4 * j + 1] * inv);
        w[1] = pack_bf16x2(oacc[dt][qc][4 * j + 2] * inv, oacc[dt][qc][4 * j + 3] * inv);
        *(u32x2*)(orow + d0) = w;
      }
  }
}

// WITH_OVL = false: plain and causal key blocks only (kstride must equal SB); the overlapping-
// block kernel is then not instantiated in the including translation unit
template <int D, int SB, int R, int KU, bool WITH_OVL = true>
hipError_t launch_tiles(int64_t B, int64_t N, int Hq, int Hkv, int topk, const void* q,
                        const void* k, const void* v, const int32_t* idx, float c, void* out,
                        float* lse, bool causal, int nkb, int kstride, hipStream_t stream) {
  const int nb = (int)(N / SB);
  const uint32_t total = (uint32_t)(B * Hq * nb * (SB / R));
#define BSATTN_BF16_LAUNCH(causal_, ovl_)                                                     \
  attn_bf16_kernel<D, SB, R, KU, causal_, ovl_><<<total, Cfg<D, R, KU>::NT, 0, stream>>>(     \
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, idx, (uint16_t*)out, lse, N, \
      Hq, Hkv, nb, topk, c, total, nkb, kstride)
  if (causal) {
    BSATTN_BF16_LAUNCH(true, false);
  } else if (kstride != SB) {
    if constexpr (WITH_OVL) BSATTN_BF16_LAUNCH(false, true);
    else return hipErrorInvalidValue;
  } else {
    BSATTN_BF16_LAUNCH(false, false);
  }
#undef BSATTN_BF16_LAUNCH
  return hipGetLastError();
}

template <int D, int SB>
hipError_t launch(int64_t B, int64_t N, int Hq, int Hkv, int topk, const void* q, const void* k,
                  const void* v, const int32_t* idx, float c, void* out, float* lse,
                  bool causal, int nkb, int kstride, hipStream_t stream) {
  if constexpr (SB == 128)
    return launch_tiles<D, SB, 128, 64>(B, N, Hq, Hkv, topk, q, k, v, idx, c, out, lse, causal,
                                        nkb, kstride, stream);
  else
    return launch_tiles<D, SB, SB, SB>(B, N, Hq, Hkv, topk, q, k, v, idx, c, out, lse, causal,
                                       nkb, kstride, stream);
}

}  // namespace

}  // namespace bsattn
