// Backward of the gathered-block attention (bf16 inputs, fp32 gradients, block 64, D 64 or
// 128) with the selected blocks held fixed.
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"): the method is
// recommended for training large models ("千亿参数大模型训练"); MSA page
// ("从M2.7到M3：多模态模型稀疏注意力架构设计与实现全解析") §4.1 checks that back-propagation
// through the sparse attention is complete. For query block i with selected keys U,
// P = softmax(scale * Q_i K_U^T) (row log-sum-exp from the forward), and the upstream dO_i:
//   dV_U += P^T dO_i,  dP = dO_i V_U^T,  dS = P * (dP - rowsum(dO_i * O_i)),
//   dQ_i = scale * dS K_U,  dK_U += scale * dS^T Q_i.
//
// Kernels:
//   index_kernel    per (batch, KV head): for every key block j the list of (query head of
//                   the group, query block) pairs that selected it, in ascending pair order
//                   (LDS counts, a scan, then the rows in order), so the key-side sums run in
//                   a fixed order and the gradients are reproducible bit for bit.
//   dq_kernel       query-major like the forward: per selected block S^T = K Q^T and
//                   dP^T = V dO^T on bf16 MFMA (A = K or V rows from LDS, B = Q^T or dO^T in
//                   registers), P^T and dS^T in fp32, dQ^T += K^T dS^T (A = K^T by LDS
//                   transpose reads, B = dS^T rounded to bf16 straight from the accumulators).
//                   It also forms Dvec[b,h,t] = sum_d dO * O (fp32) of its rows and stores it
//                   for dkv_kernel.
//   dkv_kernel      key-major: one work-group per (batch, KV head, key block) keeps K and V rows
//                   of its keys in registers (B operands) and walks its pair list: S = Q K^T,
//                   dP = dO V^T (A = Q or dO rows from LDS), P and dS in fp32, then
//                   dV^T += dO^T P and dK^T += Q^T dS (A = dO^T, Q^T by transpose reads,
//                   B = P, dS rounded to bf16 from the accumulators). No atomics.
// Layout conventions follow the forward kernel: 32x32 MFMA accumulators (register r, lane l:
// row 8(r/4) + 4(l/32) + r%4, column l%32), 16-key (or 16-query) k-steps whose 16 slots are
// matched to {4h..4h+3, 8+4h..8+4h+3} on both operands, tiles [64][D] bf16 in LDS with the
// 16-byte chunk c of row r at chunk c ^ f(r): f(r) = 4((r>>1)&1) + ((r>>2)&3) at D = 64 and
// 4(r&3) + ((r>>2)&3) at D = 128, which keeps row reads (16 rows per clock), transpose reads
// (4 rows x 64 bytes per clock) and row-major stores on distinct banks of gfx950's 64-bank LDS.
// Causal option: query block i reads its first min(topk, i+1) entries (each in [0, i]) and in
// its own block keys after the query get weight 0; the dS of masked pairs is 0.
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBlk = 64;                      // block size of this backward
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 64) return c ^ (4 * ((r >> 1) & 1) + ((r >> 2) & 3));
  else return c ^ (4 * (r & 3) + ((r >> 2) & 3));
}

__device__ __forceinline__ s16x4 ds_read_tr16(const char* lds_bytes) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_void*)(lds_bytes));
}

// vmcnt(0) only (expcnt and lgkmcnt left free), gfx9 s_waitcnt encoding
__device__ __forceinline__ void wait_vmcnt0() {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

// One [64][D] bf16 tile moved from memory straight into LDS with global_load_lds_dwordx4
// (lane l of an instruction fills bytes [16l, 16l+16) of a 1 KiB span): the chunk at
// position p of tile row r is fetched from the row's chunk swz(r, p), which gives the
// swizzled layout above. The waves of the work-group split the spans; the transfers come
// from inline asm, so the waits before the tile is read are placed by hand.
template <int D, int NT>
struct TileDma {
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int SPW = kBlk * CH / 64 / (NT / kWave);   // spans per wave
  static_assert(SPW == 4 || SPW == 8, "the transfer sequences issue 4 or 8 spans");
  uint32_t goff[SPW];                                // source byte offsets in the tile
  __device__ __forceinline__ void init(int64_t rstride, int tid) {
    const int wave = tid / kWave, lane = tid % kWave;
#pragma unroll
    for (int x = 0; x < SPW; ++x) {
      const int pos = (wave * SPW + x) * kWave + lane;
      const int r = pos / CH, c = pos % CH;
      goff[x] = (uint32_t)((r * rstride + 8 * swz<D>(r, c)) * 2);
    }
  }
  // rows row0.. of a [*, H, D] tensor (head offset folded into base) into dst
  __device__ __forceinline__ void issue(const uint16_t* base, int64_t row0, int64_t rstride,
                                        char* dst, int tid) const {
    const int wave = tid / kWave;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void*)dst + wave * SPW * 1024);
    const uint64_t sb = (uint64_t)(uintptr_t)(base + row0 * rstride);
    const char* src = (const char*)(uintptr_t)(
        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sb) |
        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sb >> 32)) << 32));
    uint32_t m0_saved;
    if constexpr (SPW == 4) {
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %6\n\t"
          "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %6\n\t"
          "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %6\n\t"
          "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, %6\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(m0_saved)
          : "s"(lds0), "v"(goff[0]), "v"(goff[1]), "v"(goff[2]), "v"(goff[3]), "s"(src)
          : "memory", "scc");
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
            "v"(goff[5]), "v"(goff[6]), "v"(goff[7]), "s"(src)
          : "memory", "scc");
    }
  }
};

// A operand (32 rows x 16 d) of a row-major tile: rows 32*t + l32, d = 16s + 8*half .. +7
template <int D>
__device__ __forceinline__ bf16x8 rows_operand(const char* tile, int t, int s, int l32, int half) {
  const int r = 32 * t + l32;
  return __builtin_bit_cast(bf16x8, *(const u32x4*)(tile + r * D * 2 + 16 * swz<D>(r, 2 * s + half)));
}

// A operand (32 d x 16 rows) of a row-major tile read transposed: d rows 32*dt + l32, rows
// 16*ps + {4h..4h+3, 8+4h..8+4h+3} (the forward's V^T reads)
template <int D>
__device__ __forceinline__ bf16x8 trans_operand(const char* tile, int dt, int ps, int lane) {
  const int half = lane >> 5;
  const int e = (lane & 15) >> 2, r = 4 * half + e;
  const int ch = 4 * dt + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const char* t = tile + 16 * ps * D * 2 + 8 * (lane & 1);
  const s16x4 a8[2] = {ds_read_tr16(t + r * D * 2 + 16 * swz<D>(r, ch)),
                       ds_read_tr16(t + (r + 8) * D * 2 + 16 * swz<D>(r + 8, ch))};
  return __builtin_bit_cast(bf16x8, a8);
}

// 8 bf16 of a global row (B operand: the lane's row, d = 16s + 8*half .. +7)
__device__ __forceinline__ bf16x8 row_chunk(const uint16_t* row, int s, int half) {
  return __builtin_bit_cast(bf16x8, *(const u32x4*)(row + 16 * s + 8 * half));
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// B operand of a 16-slot k-step from two 32-row accumulator tiles: k-step ps covers
// accumulator tile ps >> 1, registers 8*(ps&1) .. +7 (slots {4h.., 8+4h..})
__device__ __forceinline__ bf16x8 pack_step(const f32x16 (&acc)[2], int ps) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = pack_bf16x2(acc[ps >> 1][8 * (ps & 1) + 2 * e], acc[ps >> 1][8 * (ps & 1) + 2 * e + 1]);
  return __builtin_bit_cast(bf16x8, w);
}


// ---------------------------------------------------------------- inverted index
constexpr int kIdxThreads = 256;

// one work-group per (b, g): counts[j] of pairs selecting key block j, offsets (exclusive
// scan, written to `offsets` [nb + 1]) and pairs in ascending (query head of the group, query
// block) order, pair = hh * nb + i, stored at seg + offsets[j] + rank
__global__ __launch_bounds__(kIdxThreads) void index_kernel(const int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ pairs,
                                                            int Hq, int Hkv, int nb, int topk,
                                                            bool causal) {
  extern __shared__ int sm[];
  int* cnt = sm;                              // [nb + 1]: counts, then offsets
  int* cur = sm + nb + 1;                     // [nb]: next free place per key block
  __shared__ int wsum[kIdxThreads / kWave];
  const int bg = blockIdx.x;
  const int b = bg / Hkv, g = bg % Hkv, G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int rows = G * nb;                    // (hh, i) rows of this group, in pair order
  const int32_t* gidx = idx + ((int64_t)b * Hq + (int64_t)g * G) * nb * topk;
  for (int j = tid; j <= nb; j += kIdxThreads) cnt[j] = 0;
  __syncthreads();
  for (int64_t e = tid; e < (int64_t)rows * topk; e += kIdxThreads) {
    const int i = (int)((e / topk) % nb), t = (int)(e % topk);
    const int used = causal && i + 1 < topk ? i + 1 : topk;
    const int j = gidx[e];
    if (t < used && (unsigned)j < (unsigned)nb) atomicAdd(&cnt[j], 1);
  }
  __syncthreads();
  // exclusive scan of cnt[0..nb) in place; cnt[nb] = total
  {
    const int per = (nb + kIdxThreads - 1) / kIdxThreads;
    const int j0 = tid * per;
    int local = 0;
    for (int j = j0; j < j0 + per && j < nb; ++j) local += cnt[j];
    int incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if ((tid & (kWave - 1)) >= o) incl += y;
    }
    if ((tid & (kWave - 1)) == kWave - 1) wsum[tid / kWave] = incl;
    __syncthreads();
    int before = incl - local;
    for (int w = 0; w < tid / kWave; ++w) before += wsum[w];
    __syncthreads();
    for (int j = j0; j < j0 + per && j < nb; ++j) {
      const int c = cnt[j];
      cnt[j] = before;
      cur[j] = before;
      before += c;
    }
    if (tid == kIdxThreads - 1) cnt[nb] = before;
  }
  __syncthreads();
  int32_t* off = offsets + (int64_t)bg * (nb + 1);
  for (int j = tid; j <= nb; j += kIdxThreads) off[j] = cnt[j];
  int32_t* seg = pairs + (int64_t)bg * rows * topk;
  // rows in order; the entries of one row name distinct blocks, so one step has no conflict
  for (int row = 0; row < rows; ++row) {
    const int i = row % nb;
    const int used = causal && i + 1 < topk ? i + 1 : topk;
    for (int t = tid; t < used; t += kIdxThreads) {
      const int j = gidx[(int64_t)row * topk + t];
      if ((unsigned)j < (unsigned)nb) seg[atomicAdd(&cur[j], 1)] = row;   // atomic: a row
    }                                                                      // may repeat j
    __syncthreads();
  }
}

// ---------------------------------------------------------------- dQ
// work-group per (b, h, query block i): 2 waves x 32 queries
template <int D, bool CAUSAL>
__global__ __launch_bounds__(128) void dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ out, const int32_t* __restrict__ idx,
    const float* __restrict__ lse, float* __restrict__ dvec, float* __restrict__ dq, int64_t N,
    int Hq, int Hkv, int nb, int topk, float c, float scale, uint32_t total_tiles) {
  constexpr int NS = D / 16, NDT = D / 32;
  // D = 64: one V buffer (24 KiB of LDS per work-group: three waves per SIMD); D = 128: two
  // (the single-buffer schedule needs more registers than two waves per SIMD allow there)
  constexpr bool kOneV = D == 64;
  __shared__ __attribute__((aligned(1024))) char Kt[2][kBlk * D * 2];
  __shared__ __attribute__((aligned(1024))) char Vt[kOneV ? 1 : 2][kBlk * D * 2];
  const uint32_t tile = xcd_remap(blockIdx.x, total_tiles);
  const int G = Hq / Hkv;
  const int i = (int)(tile % nb);
  uint32_t rest = tile / nb;
  const int hh = (int)(rest % G);
  rest /= G;
  const int g = (int)(rest % Hkv);
  const int b = (int)(rest / Hkv);
  const int h = g * G + hh;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t qrs = (int64_t)Hq * D, krs = (int64_t)Hkv * D;
  const int qloc = 32 * wave + l32;           // query row of this lane's column, in the block
  const int64_t qrow = (int64_t)b * N + (int64_t)i * kBlk + qloc;

  bf16x8 qf[NS], gf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = row_chunk(q + qrow * qrs + (int64_t)h * D, s, half);
    gf[s] = row_chunk(dout + qrow * qrs + (int64_t)h * D, s, half);
  }
  const int64_t rowid = ((int64_t)b * Hq + h) * N + (int64_t)i * kBlk + qloc;
  const float l2 = lse[rowid] * kLog2e;       // log2-sum-exp of the row
  // Dvec of the row, rowsum(dO * O) in fp32: the two lanes of the row take the same 8-element
  // chunks as their dO operands; stored for dkv_kernel, which runs after this kernel
  float ddp = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bf16x8 o8 = row_chunk(out + qrow * qrs + (int64_t)h * D, s, half);
#pragma unroll
    for (int e = 0; e < 8; ++e) ddp = __builtin_fmaf((float)gf[s][e], (float)o8[e], ddp);
  }
  const float dd = ddp + __shfl_xor(ddp, 32);
  if (half == 0) dvec[rowid] = dd;
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  const int32_t* myidx = idx + (((int64_t)b * Hq + h) * nb + i) * topk;
  const int kcount = CAUSAL && i + 1 < topk ? i + 1 : topk;
  const unsigned klim = CAUSAL ? (unsigned)(i + 1) : (unsigned)nb;
  const uint16_t* kb0 = k + (int64_t)b * N * krs + (int64_t)g * D;
  const uint16_t* vb0 = v + (int64_t)b * N * krs + (int64_t)g * D;

  // an out-of-range entry is never read (the forward gave its rows NaN): block 0 stands in
  // and the step is skipped. The K tile of step t + 1 moves into the other K buffer during
  // the whole of step t; V, read only by the dP product, goes into the other V buffer too
  // (D = 128) or into its single buffer once every wave has formed dP (D = 64).
  TileDma<D, 128> tk;
  tk.init(krs, tid);
  auto row0 = [&](int jj) -> int64_t { return (unsigned)jj < klim ? (int64_t)jj * kBlk : 0; };
  if (kcount > 0) {
    tk.issue(kb0, row0(myidx[0]), krs, Kt[0], tid);
    tk.issue(vb0, row0(myidx[0]), krs, Vt[0], tid);
  }
  // one step; the buffer index is a compile-time constant (the loop below takes steps two at
  // a time), so the LDS read addresses stay fixed and the buffer goes into the offset field
  auto kv_step = [&](int t, auto buf) {
    constexpr int cur = decltype(buf)::value;
    const int j = myidx[t];
    const bool more = t + 1 < kcount;
    wait_vmcnt0();                            // this wave's transfers of step t
    __syncthreads();                          // every wave's landed; step t-1 done everywhere
    if (more) {
      tk.issue(kb0, row0(myidx[t + 1]), krs, Kt[cur ^ 1], tid);
      if (!kOneV) tk.issue(vb0, row0(myidx[t + 1]), krs, Vt[kOneV ? 0 : cur ^ 1], tid);
    }
    const char* Kc = Kt[cur];
    const char* Vc = Vt[kOneV ? 0 : cur];
    if ((unsigned)j >= klim) {                // uniform: the next V tile still moves
      if (kOneV) {
        __syncthreads();
        if (more) tk.issue(vb0, row0(myidx[t + 1]), krs, Vt[0], tid);
      }
      return;
    }
    f32x16 st[2], dpt[2];                     // S^T and dP^T: rows = 64 keys, cols = queries
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) { st[kt][r] = 0.f; dpt[kt][r] = 0.f; }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        st[kt] = mfma(rows_operand<D>(Kc, kt, s, l32, half), qf[s], st[kt]);
        dpt[kt] = mfma(rows_operand<D>(Vc, kt, s, l32, half), gf[s], dpt[kt]);
      }
    }
    if (kOneV) {
      __syncthreads();                        // every wave has read V(t)
      if (more) tk.issue(vb0, row0(myidx[t + 1]), krs, Vt[0], tid);
    }
    // dS^T = P^T (dP^T - Dvec), P^T = exp2(c s - lse2); masked keys give 0
    const bool own = CAUSAL && j == i;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kt][r], c, -l2));
        if (own && key > qloc) p = 0.f;
        dpt[kt][r] = p * (dpt[kt][r] - dd);
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const bf16x8 bds = pack_step(dpt, ps);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] = mfma(trans_operand<D>(Kc, dt, ps, lane), bds, acc[dt]);
    }
  };
  for (int t = 0; t < kcount; t += 2) {
    kv_step(t, std::integral_constant<int, 0>{});
    if (t + 1 < kcount) kv_step(t + 1, std::integral_constant<int, 1>{});
  }
  // dQ = scale * (dQ^T)^T: lane holds d = 32dt + 8(r/4) + 4*half + r%4 of query qloc
  float* drow = dq + qrow * qrs + (int64_t)h * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      f32x4 w;
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = acc[dt][4 * jj + u] * scale;
      *(f32x4*)(drow + 32 * dt + 8 * jj + 4 * half) = w;
    }
}

// ---------------------------------------------------------------- dK, dV
// work-group per (b, g, key block j): 2 waves x 32 keys
template <int D, bool CAUSAL>
// (D = 64) two waves per SIMD is what its registers allow anyway; saying so lets the scheduler use
// up to 256 registers for earlier operand reads (1 % faster, identical gradients)
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1))) void dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ dvec,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs,
    float* __restrict__ dk, float* __restrict__ dv, int64_t N, int Hq, int Hkv, int nb,
    int topk, float c, float scale, uint32_t total_tiles) {
  constexpr int NS = D / 16, NDT = D / 32;
  __shared__ __attribute__((aligned(1024))) char Qt[2][kBlk * D * 2];   // two buffers each
  __shared__ __attribute__((aligned(1024))) char Gt[2][kBlk * D * 2];   // dO tiles
  __shared__ __attribute__((aligned(16))) float l2s[2][kBlk];
  __shared__ __attribute__((aligned(16))) float dds[2][kBlk];      // -Dvec of the rows
  const uint32_t tile = xcd_remap(blockIdx.x, total_tiles);
  const int j = (int)(tile % nb);
  const int bg = (int)(tile / nb);
  const int b = bg / Hkv, g = bg % Hkv, G = Hq / Hkv;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t qrs = (int64_t)Hq * D, krs = (int64_t)Hkv * D;
  const int kloc = 32 * wave + l32;           // key of this lane's column, in the block
  const int64_t krow = (int64_t)b * N + (int64_t)j * kBlk + kloc;

  bf16x8 kf[NS], vf[NS];                      // B operands: K^T, V^T (lane = key)
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kf[s] = row_chunk(k + krow * krs + (int64_t)g * D, s, half);
    vf[s] = row_chunk(v + krow * krs + (int64_t)g * D, s, half);
  }
  f32x16 dka[NDT], dva[NDT];                  // dK^T, dV^T: rows = d, cols = keys
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dka[dt][r] = 0.f; dva[dt][r] = 0.f; }

  const int32_t* off = offsets + (int64_t)bg * (nb + 1);
  const int32_t* seg = pairs + (int64_t)bg * G * nb * topk;
  const int p0 = off[j], p1 = off[j + 1];
  // the tiles of pair p + 1 move into the other LDS buffers while pair p is multiplied (one
  // barrier per pair); a pair value out of range (only possible for idx rows with repeated
  // blocks) is skipped, pair 0 standing in
  TileDma<D, 128> tq;
  tq.init(qrs, tid);
  float l2n = 0.f, ddn = 0.f;
  auto fetch = [&](int p, int buf) {
    int row = seg[p];
    if ((unsigned)row >= (unsigned)(G * nb)) row = 0;
    const int h = g * G + row / nb, i = row % nb;
    const int64_t r0 = (int64_t)b * N + (int64_t)i * kBlk;
    tq.issue(q + (int64_t)h * D, r0, qrs, Qt[buf], tid);
    tq.issue(dout + (int64_t)h * D, r0, qrs, Gt[buf], tid);
    if (tid < kBlk) {
      const int64_t rid = ((int64_t)b * Hq + h) * N + (int64_t)i * kBlk + tid;
      l2n = lse[rid] * kLog2e;
      ddn = dvec[rid];
    }
  };
  if (p0 < p1) fetch(p0, 0);
  // one pair; the buffer index is a compile-time constant (the loop below takes pairs two at a
  // time), so the LDS read addresses stay fixed and the buffer goes into the offset field
  auto pair_step = [&](int p, auto buf) {
    constexpr int cur = decltype(buf)::value;
    const int row = seg[p];                   // hh * nb + i
    wait_vmcnt0();                            // this wave's transfers and loads for pair p
    if (tid < kBlk) { l2s[cur][tid] = l2n; dds[cur][tid] = -ddn; }
    __syncthreads();                          // every wave's landed; pair p-1 done everywhere
    if (p + 1 < p1) fetch(p + 1, cur ^ 1);
    if ((unsigned)row >= (unsigned)(G * nb)) return;     // uniform
    const int i = row % nb;
    const char* Qc = Qt[cur];
    const char* Gc = Gt[cur];
    const float* l2c = l2s[cur];
    const float* ddc = dds[cur];
    // S and dP: rows = 64 queries, cols = keys. The dP accumulators start at -Dvec of their
    // rows (registers 4*r4 .. 4*r4+3 hold rows q0 .. q0+3: one 16-byte read per 4 rows), so the
    // products leave dP - Dvec in them
    f32x16 sa[2], dpa[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 d4 = *(const f32x4*)(ddc + 32 * qt + 8 * r4 + 4 * half);
#pragma unroll
        for (int u = 0; u < 4; ++u) { sa[qt][4 * r4 + u] = 0.f; dpa[qt][4 * r4 + u] = d4[u]; }
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sa[qt] = mfma(rows_operand<D>(Qc, qt, s, l32, half), kf[s], sa[qt]);
        dpa[qt] = mfma(rows_operand<D>(Gc, qt, s, l32, half), vf[s], dpa[qt]);
      }
    }
    const bool own = CAUSAL && i == j;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int q0 = 32 * qt + 8 * r4 + 4 * half;
        const f32x4 l4 = *(const f32x4*)(l2c + q0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * r4 + u;
          float pp = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[qt][r], c, -l4[u]));
          if (own && kloc > q0 + u) pp = 0.f;
          sa[qt][r] = pp;                                 // P
          dpa[qt][r] = pp * dpa[qt][r];                   // dS = P (dP - Dvec)
        }
      }
    // dV^T += dO^T P, dK^T += Q^T dS (k-steps over the 64 queries)
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const bf16x8 bp = pack_step(sa, ps), bs = pack_step(dpa, ps);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        dva[dt] = mfma(trans_operand<D>(Gc, dt, ps, lane), bp, dva[dt]);
        dka[dt] = mfma(trans_operand<D>(Qc, dt, ps, lane), bs, dka[dt]);
      }
    }
  };
  for (int p = p0; p < p1; p += 2) {
    pair_step(p, std::integral_constant<int, 0>{});
    if (p + 1 < p1) pair_step(p + 1, std::integral_constant<int, 1>{});
  }
  float* krow_dk = dk + krow * krs + (int64_t)g * D;
  float* krow_dv = dv + krow * krs + (int64_t)g * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      f32x4 wk, wv;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wk[u] = dka[dt][4 * jj + u] * scale;
        wv[u] = dva[dt][4 * jj + u];
      }
      *(f32x4*)(krow_dk + 32 * dt + 8 * jj + 4 * half) = wk;
      *(f32x4*)(krow_dv + 32 * dt + 8 * jj + 4 * half) = wv;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(int64_t B, int64_t N, int Hq, int Hkv, int topk, const void* q,
                      const void* k, const void* v, const int32_t* idx, const void* out,
                      const void* dout, const float* lse, float scale, float* dq, float* dk,
                      float* dv, float* dvec, int32_t* offsets, int32_t* pairs,
                      hipStream_t stream) {
  const int nb = (int)(N / kBlk);
  const float c = (float)((double)scale * 1.4426950408889634);
  const size_t lds = (size_t)(2 * nb + 1) * sizeof(int);
  index_kernel<<<(unsigned)(B * Hkv), kIdxThreads, lds, stream>>>(idx, offsets, pairs, Hq, Hkv,
                                                                  nb, topk, CAUSAL);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t tq = (uint32_t)(B * Hq * nb);
  dq_kernel<D, CAUSAL><<<tq, 128, 0, stream>>>(
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
      (const uint16_t*)out, idx, lse, dvec, dq, N, Hq, Hkv, nb, topk, c, scale, tq);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t tk = (uint32_t)(B * Hkv * nb);
  dkv_kernel<D, CAUSAL><<<tk, 128, 0, stream>>>(
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, lse,
      dvec, offsets, pairs, dk, dv, N, Hq, Hkv, nb, topk, c, scale, tk);
  return hipGetLastError();
}

}  // namespace

namespace {

// 128-token blocks as 64-token blocks: query block i (128 tokens) becomes the 64-token blocks
// 2i and 2i+1, each selected block j the 64-token blocks 2j and 2j+1 (the key set of every
// query is unchanged, so the gradients are those of the 128-token selection). Causal rows of
// the first half leave out 2i+1, the second half of their own block, which lies after each of
// their queries. An entry out of range becomes two out-of-range entries (skipped like it).
// One thread per 64-token row.
__global__ __launch_bounds__(256) void expand_idx128_kernel(const int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ idx64,
                                                            int64_t rows, int nb, int topk,
                                                            bool causal) {
  const int64_t r64 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r64 >= 2 * rows) return;
  const int64_t r = r64 >> 1;
  const int part = (int)(r64 & 1), i = (int)(r % nb);
  const int32_t* src = idx + r * topk;
  int32_t* dst = idx64 + r64 * 2 * topk;
  const int used = causal && i + 1 < topk ? i + 1 : topk;
  int p = 0;
  for (int t = 0; t < used; ++t) {
    const int j = src[t];
    if ((unsigned)j >= (unsigned)nb) {
      dst[p++] = -1;
      dst[p++] = -1;
    } else {
      dst[p++] = 2 * j;
      if (!(causal && part == 0 && j == i)) dst[p++] = 2 * j + 1;
    }
  }
  for (; p < 2 * topk; ++p) dst[p] = -1;
}

}  // namespace

bool attn_bwd_supported(int dtype_kind, int D, int block) {
  return dtype_kind == 1 && (D == 64 || D == 128) && (block == kBlk || block == 2 * kBlk);
}

size_t attn_bwd_workspace_bytes(int64_t B, int64_t N, int Hq, int Hkv, int block, int topk) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  if (block == 2 * kBlk)                     // the 64-token form, then its index rows
    return attn_bwd_workspace_bytes(B, N, Hq, Hkv, kBlk, 2 * topk) +
           al((size_t)B * Hq * (N / kBlk) * 2 * topk * sizeof(int32_t));
  const int64_t nb = N / block;
  return al((size_t)B * Hq * N * sizeof(float)) +                  // Dvec
         al((size_t)B * Hkv * (nb + 1) * sizeof(int32_t)) +        // offsets
         al((size_t)B * Hq * nb * topk * sizeof(int32_t));         // pairs
}

hipError_t launch_expand_idx128(int64_t rows, int nb, int topk, bool causal, const int32_t* idx,
                                int32_t* idx64, hipStream_t stream) {
  expand_idx128_kernel<<<(unsigned)((2 * rows + 255) / 256), 256, 0, stream>>>(idx, idx64, rows,
                                                                            nb, topk, causal);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(int64_t B, int64_t N, int Hq, int Hkv, int D, int topk, bool causal,
                           const void* q, const void* k, const void* v, const int32_t* idx,
                           const void* out, const void* dout, const float* lse, float scale,
                           float* dq, float* dk, float* dv, void* workspace,
                           hipStream_t stream) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t nb = N / kBlk;
  char* w = (char*)workspace;
  float* dvec = (float*)w;
  int32_t* offsets = (int32_t*)(w + al((size_t)B * Hq * N * sizeof(float)));
  int32_t* pairs = (int32_t*)((char*)offsets + al((size_t)B * Hkv * (nb + 1) * sizeof(int32_t)));
  if (D == 64)
    return causal ? launch_bwd<64, true>(B, N, Hq, Hkv, topk, q, k, v, idx, out, dout, lse, scale,
                                         dq, dk, dv, dvec, offsets, pairs, stream)
                  : launch_bwd<64, false>(B, N, Hq, Hkv, topk, q, k, v, idx, out, dout, lse, scale,
                                          dq, dk, dv, dvec, offsets, pairs, stream);
  return causal ? launch_bwd<128, true>(B, N, Hq, Hkv, topk, q, k, v, idx, out, dout, lse, scale,
                                        dq, dk, dv, dvec, offsets, pairs, stream)
                : launch_bwd<128, false>(B, N, Hq, Hkv, topk, q, k, v, idx, out, dout, lse, scale,
                                         dq, dk, dv, dvec, offsets, pairs, stream);
}

}  // namespace bsattn
