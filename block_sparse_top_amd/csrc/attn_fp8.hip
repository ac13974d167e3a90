// Step 4 for OCP fp8 (e4m3) inputs: attention over the gathered selected blocks on the gfx950
// fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, unit block scales), fp32 accumulation, bf16
// output.
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"), "SparseFormer 注意力
// 实现" step 3 (attention over the selected blocks, scale 1/sqrt(D)); its closing section names
// FP8 tensor cores for this workload. MSA page ("从M2.7到M3：多模态模型稀疏注意力架构设计与实现全解析")
// §2.1 (Softmax(Mask(QK^T/sqrt(d_k)))V), §3.1 (GQA).
//
// Values are e4m3 codes times per-tensor descales dq, dk, dv. The kernel multiplies codes:
// S^T = K Q^T on codes, z = s * c with c = scale*log2(e)*dq*dk, weights p = exp2(z - m + 7)
// quantised to e4m3 for the PV product (m = the row's reference max, so p <= 2^8 < 448),
// O^T += V^T P^T on codes, and out = O * dv / l. Unlike the bf16 kernel the reference must
// track the row max (an e4m3 weight needs a bounded range): a block whose max exceeds the
// reference by more than one exp2 unit moves it up and rescales O and l.
//
// Work split and data movement follow the bf16 kernel: one work-group per (batch, query head,
// query block), 32 query rows per wave, K and V tiles [BLK][128] bytes moved into LDS with
// global_load_lds_dwordx4 from inline asm (hand-placed waits), S^T from K rows (two 16-byte
// LDS reads per operand), V^T operands from ds_read_b64_tr_b8 transpose reads (in each 16-lane
// group, output lane i takes byte i%8 of the 8 bytes named by lane 2e + i/8, e = 0..7). The
// 32 k-slots of lane half h are keys 32kt + 8j + 4h + t (kt<2, j<4, t<4) on both operands of
// the PV product: exactly the keys the S^T accumulators give that lane. 16-byte chunk c of
// tile row r sits at chunk c ^ f(r), f(r) = 2((r>>1)&1) + 4((r>>3)&1) + ((r>>2)&1). gfx950's
// LDS has 64 banks of 4 bytes and a 128-byte row fills half a bank line: the K row reads
// (16 lanes per clock, rows 0..15) see f take all 8 values on the even and on the odd rows,
// and the V transpose reads (32 lanes per clock: rows {0,2,8,10} or {4,6,12,14} and the odd
// ones, 2 chunks each) see f>>1 take 4 distinct values, so both cover the 64 banks once.
//
// Causal variant (template flag): query block i reads the first min(topk, i+1) entries of its
// row, each in [0, i]; in its own block the scores of keys after the query are -inf before
// the row maximum and the weights.
// Overlapping key blocks (template flag; the MSA page's §5.3): block j's tile starts at
// key_tile_start and its first key_tile_skip keys score -inf (at least one key of every tile
// counts, so the row maximum of a tile is finite).
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = 128;                       // head dimension (bytes per fp8 row)
constexpr float kGrow = 1.0f;                 // reference moves when a block max exceeds it by this
constexpr float kBias = 7.0f;                 // weights exp2(z - m + 7) <= 2^8

template <int BLK>
struct Cfg8 {
  static constexpr int NW = BLK / 32;         // waves, 32 query rows each
  static constexpr int NT = NW * kWave;
  static constexpr int TILE = BLK * kD;       // bytes of one K or V tile
  static constexpr int DMA = TILE / 1024 / NW;  // = 4
  static constexpr int NKT = BLK / 32;        // 32-key sub-tiles
  static constexpr int NS = kD / 64;          // k-steps of Q K^T (64 bytes each)
  static constexpr int NDT = kD / 32;         // 32-row d tiles of O^T
  static constexpr int NKS = BLK / 64;        // k-steps of V^T P^T (64 keys each)
  static_assert(DMA == 4, "transfer sequence below issues 4 spans of 1 KiB");
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ int swz8(int r) {
  return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2) | ((r >> 2) & 1);
}

__device__ __forceinline__ i32x2 ds_read_tr8(const char* lds_bytes) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(lds_void*)(lds_bytes));
}

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // format 0 (e4m3) for both operands, e8m0 scale 127 (x1) for both
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int BLK, bool CAUSAL, bool OVL>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(BLK == 64 ? 3 : 2))) void attn_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ out, float* __restrict__ lse,
    int64_t N, int Hq, int Hkv, int nb, int topk, float c, float dv, uint32_t total_tiles,
    int nkb, int kstride) {
  using C = Cfg8<BLK>;
  __shared__ __attribute__((aligned(1024))) char Kl[C::TILE];
  __shared__ __attribute__((aligned(1024))) char Vl[C::TILE];
  __shared__ uint32_t chosen[OVL ? kMaxKeyBlocks / 32 : 1];   // OVL: the row's key blocks

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
  const int64_t qrs = (int64_t)Hq * kD;        // token stride of q/out (elements)
  const int64_t krs = (int64_t)Hkv * kD;       // token stride of k/v (bytes)

  // Q^T as B operands: lane holds q[row][64s + 32*half .. +31]
  const int64_t qrow = (int64_t)b * N + (int64_t)i * BLK + 32 * wave + l32;
  i32x8 qf[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
    const uint8_t* p = q + qrow * qrs + (int64_t)h * kD + 64 * s + 32 * half;
    const u32x4 lo = *(const u32x4*)p, hi = *(const u32x4*)(p + 16);
    // Q must have landed before the first transfer: the hand-placed vmcnt waits in the loop
    // count transfers only (the empty asm consumes the loaded registers here)
    asm volatile("" ::"v"(lo), "v"(hi));
    qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }

  const int32_t* myidx = idx + (((int64_t)b * Hq + h) * nb + i) * topk;
  const char* kbase0 = (const char*)(k + (int64_t)b * N * krs + (int64_t)g * kD);
  const char* vbase0 = (const char*)(v + (int64_t)b * N * krs + (int64_t)g * kD);

  uint32_t goff[C::DMA];
#pragma unroll
  for (int x = 0; x < C::DMA; ++x) {
    const int pos = (wave * C::DMA + x) * 64 + lane;         // 16-byte chunk in the tile
    const int r = pos / 8, p = pos % 8;
    goff[x] = (uint32_t)(r * krs + (p ^ swz8(r)) * 16);
  }
  bool bad = false;
  const int kcount = CAUSAL && i + 1 < topk ? i + 1 : topk;   // entries of the row used
  const unsigned klim = CAUSAL ? (unsigned)(i + 1) : (unsigned)(OVL ? nkb : nb);
  auto tile_base = [&](int kb) -> int64_t {
    if ((unsigned)kb >= klim) { bad = true; kb = 0; }
    return (OVL ? key_tile_start(kb, kstride, BLK, N) : (int64_t)kb * BLK) * krs;
  };
  auto skip_of = [&](int kb) -> int {          // OVL: leading keys of kb's tile left out
    if (!OVL || (unsigned)kb >= klim) return 0;
    return key_tile_skip(kb, kstride, BLK, N, is_selected(chosen, kb - 1));
  };
  // transfers from inline asm: the compiler's wait-count pass adds no vmcnt(0) before the
  // LDS reads; each wave issues exactly DMA transfers per tile and no other vector-memory
  // instruction inside the loop. M0 (the LDS destination) is saved and restored around them.
  auto dma = [&](const char* src_base, char* dst) {
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void*)dst + wave * C::DMA * 1024);
    uint32_t m0_saved;
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
  };

  // LDS read offsets: K rows 32kt + l32, chunks 4s + 2*half (+1)
  const int fk = swz8(l32);
  int koff[C::NS][2];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
    koff[s][0] = l32 * kD + 16 * ((4 * s + 2 * half) ^ fk);
    koff[s][1] = l32 * kD + 16 * ((4 * s + 2 * half + 1) ^ fk);
  }
  // V transpose reads: source lane j of 16-lane group grp names row 8(j/8) + 4*half + (j/2)%4
  // (+16 per read), column 32dt + 16(grp%2) + 8(j%2)
  int voff[C::NDT];
  {
    const int j = lane & 15, grp = lane >> 4;
    const int r = 8 * (j >> 3) + 4 * half + ((j >> 1) & 3);
    const int f = swz8(r);
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
      voff[dt] = r * kD + 16 * ((2 * dt + (grp & 1)) ^ f) + 8 * (j & 1);
  }

  f32x16 oacc[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m = -__builtin_inff();                // reference (exp2 domain) of this lane's row
  float lsum = 0.f;

  if (OVL) mark_selected(chosen, myidx, kcount, nkb, tid, C::NT);
  int kb_cur = myidx[0];
  int skip_cur = skip_of(kb_cur);
  {
    const int64_t tb = tile_base(kb_cur);
    dma(kbase0 + tb, Kl);
    dma(vbase0 + tb, Vl);
  }

  for (int t = 0; t < kcount; ++t) {
    const bool more = t + 1 < kcount;
    const int kb_next = more ? myidx[t + 1] : 0;
    const int64_t tb_next = more ? tile_base(kb_next) : 0;
    const int skip_next = OVL && more ? skip_of(kb_next) : 0;

    wait_vmcnt<C::DMA>();
    if (C::NW > 1) __syncthreads();
    i32x8 ka[C::NKT][C::NS];
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        const u32x4 lo = *(const u32x4*)(Kl + kt * 32 * kD + koff[s][0]);
        const u32x4 hi = *(const u32x4*)(Kl + kt * 32 * kD + koff[s][1]);
        ka[kt][s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
    wait_lgkmcnt0();
    if (C::NW > 1) __syncthreads();
    if (more) dma(kbase0 + tb_next, Kl);

    f32x16 sacc[C::NKT];
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < C::NS; ++s) sacc[kt] = mfma8(ka[kt][s], qf[s], sacc[kt]);
    }
    if (CAUSAL && kb_cur == i) {               // own block: keys after the query get -inf
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key > 32 * wave + l32) sacc[kt][r] = -__builtin_inff();
        }
    }
    if (OVL && skip_cur > 0) {                 // keys before the block or held by block kb-1
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key < skip_cur) sacc[kt][r] = -__builtin_inff();
        }
    }

    // reference: follow the row max (lane pair l, l^32 shares one row)
    float mt = sacc[0][0];
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kt][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32)) * c;
    if (__ballot(mt > m + kGrow)) {
      const float m_new = fmaxf(m, mt);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);   // 0 on the first block
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m = m_new;
    }
    const float mb = m - kBias;
    i32x8 pb[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const f32x16& sa = sacc[2 * ks + (w >> 2)];
        float p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[4 * (w & 3) + u], c, -mb));
          lsum += p[u];
        }
        int dw = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        dw = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], dw, true);
        pb[ks][w] = dw;
      }

    if (more) wait_vmcnt<C::DMA>(); else wait_vmcnt<0>();
    if (C::NW > 1) __syncthreads();
    i32x8 va[C::NKS][C::NDT];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        i32x2 part[4];
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
          part[mm] = ds_read_tr8(Vl + (16 * (4 * ks + mm)) * kD + voff[dt]);
        va[ks][dt] = i32x8{part[0][0], part[0][1], part[1][0], part[1][1],
                           part[2][0], part[2][1], part[3][0], part[3][1]};
      }
    wait_lgkmcnt0();
    if (C::NW > 1) __syncthreads();
    if (more) dma(vbase0 + tb_next, Vl);

#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) oacc[dt] = mfma8(va[ks][dt], pb[ks], oacc[dt]);
    kb_cur = kb_next;
    if (OVL) skip_cur = skip_next;
  }

  const float l_all = lsum + __shfl_xor(lsum, 32);
  const float inv = bad ? __builtin_nanf("") : dv / l_all;
  if (lse && half == 0)                        // natural log-sum-exp (weights carry 2^kBias)
    lse[((int64_t)b * Hq + h) * N + (qrow - (int64_t)b * N)] =
        bad ? __builtin_nanf("") : (m - kBias + log2f(l_all)) * 0.6931471805599453f;
  uint16_t* orow = out + qrow * qrs + (int64_t)h * kD;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d0 = 32 * dt + 8 * jj + 4 * half;
      u32x2 w;
      w[0] = pack_bf16x2(oacc[dt][4 * jj + 0] * inv, oacc[dt][4 * jj + 1] * inv);
      w[1] = pack_bf16x2(oacc[dt][4 * jj + 2] * inv, oacc[dt][4 * jj + 3] * inv);
      *(u32x2*)(orow + d0) = w;
    }
}

template <int BLK>
hipError_t launch(int64_t B, int64_t N, int Hq, int Hkv, int topk, const void* q, const void* k,
                  const void* v, const int32_t* idx, float c, float dv, void* out, float* lse,
                  bool causal, int nkb, int kstride, hipStream_t stream) {
  const int nb = (int)(N / BLK);
  const uint32_t total = (uint32_t)(B * Hq * nb);
#define BSATTN_FP8_LAUNCH(causal_, ovl_)                                                      \
  attn_fp8_kernel<BLK, causal_, ovl_><<<total, Cfg8<BLK>::NT, 0, stream>>>(                    \
      (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, idx, (uint16_t*)out, lse, N, Hq, \
      Hkv, nb, topk, c, dv, total, nkb, kstride)
  if (causal)
    BSATTN_FP8_LAUNCH(true, false);
  else if (kstride != BLK)
    BSATTN_FP8_LAUNCH(false, true);
  else
    BSATTN_FP8_LAUNCH(false, false);
#undef BSATTN_FP8_LAUNCH
  return hipGetLastError();
}

}  // namespace

bool attn_fp8_supported(int D, int block) { return D == 128 && (block == 64 || block == 128); }

hipError_t launch_attn_fp8(int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                           const void* q, const void* k, const void* v, const int32_t* idx,
                           float scale, const float* descale_qkv, void* out, float* lse,
                           bool causal, int key_stride, int64_t nkb, hipStream_t stream) {
  (void)D;
  const float c = (float)((double)scale * 1.4426950408889634 * (double)descale_qkv[0] *
                          (double)descale_qkv[1]);
  const float dv = descale_qkv[2];
  if (block == 64)
    return launch<64>(B, N, Hq, Hkv, topk, q, k, v, idx, c, dv, out, lse, causal, (int)nkb,
                      key_stride, stream);
  return launch<128>(B, N, Hq, Hkv, topk, q, k, v, idx, c, dv, out, lse, causal, (int)nkb,
                     key_stride, stream);
}

}  // namespace bsattn
