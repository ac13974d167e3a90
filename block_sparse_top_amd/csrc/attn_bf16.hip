// Step 4: attention over the gathered selected blocks, bf16 inputs, bf16 MFMA (gfx950).
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"), section
// "SparseFormer 注意力实现", step 3: attention is computed only over the selected blocks with
// scale 1/sqrt(D); MSA page ("从M2.7到M3：多模态模型稀疏注意力架构设计与实现全解析") §2.1:
// Softmax(Mask(Q K^T / sqrt(d_k))) V with a block mask, §2.2: full attention inside the chosen
// blocks, §3.1: GQA. The softmax is exact: it is evaluated online over the k selected key
// blocks with a reference maximum and a normaliser in fp32.
//
// One work-group owns one query block (BLK rows) of one (batch, query head); each of its
// BLK/32 waves owns 32 query rows. Per selected key block the work-group stages K and V
// [BLK][D] row-major in LDS (two buffers: the next block's global loads are issued before the
// current block's math), then each wave computes
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = its Q^T in registers)
//   P^T = exp2(c*S^T - c*m)   (c = scale*log2(e), m = reference max of the query row)
//   O^T += V^T P^T (A = V^T via ds_read_b64_tr_b16 transpose reads of the row-major V tile,
//                   B = P^T built straight from the S^T accumulators)
// Working on the transposed products keeps each query's key scores in two lanes (l, l^32),
// and the score accumulators are already in the B-operand layout of the next product: the 16
// k-slots of a step are matched to keys {4h..4h+3, 8+4h..8+4h+3} on both operands.
//
// Reference maximum: it is the query row's max over the first selected block and is moved
// only when a later block would make some weight exp2(c*s - c*m) exceed 2^32 (checked on the
// per-lane block sum). Then the row max is recomputed, O and l are rescaled and the block's
// weights are recomputed. Because O and l always use the same reference, O/l is exact; the
// common case needs no max, no rescale and no cross-lane traffic. The normaliser is summed
// from the bf16-rounded weights (v_dot2c_f32_bf16), i.e. from exactly the weights the PV
// product uses.
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

constexpr float kRescaleSum = 4294967296.0f;    // 2^32

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int D, int BLK>
struct Cfg {
  static constexpr int NW = BLK / 32;          // waves (32 query rows each)
  static constexpr int NT = NW * kWave;        // threads
  static constexpr int KS = D + 8;             // K row stride in LDS (bf16): b128 reads
  static constexpr int VS = D + 16;            // V row stride in LDS (bf16): transpose reads
  static constexpr int K_ELEMS = BLK * KS;
  static constexpr int V_ELEMS = BLK * VS;
  static constexpr int CH = BLK * D / 8 / NT;  // 16-byte chunks per thread per tile (= D/16)
  static constexpr int NKT = BLK / 32;         // 32-key sub-tiles per block
  static constexpr int NS = D / 16;            // k-steps of Q K^T
  static constexpr int NDT = D / 32;           // 32-row d tiles of O^T
  static constexpr int NPS = BLK / 16;         // k-steps of V^T P^T
};

__device__ __forceinline__ s16x4 ds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) void*)(p));
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, uint16_t* __restrict__ out,
    int64_t N, int Hq, int Hkv, int nb, int topk, float c, uint32_t total_tiles) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (C::K_ELEMS + C::V_ELEMS)];
  uint16_t* Ks = lds;                          // [2][BLK][KS]
  uint16_t* Vs = lds + 2 * C::K_ELEMS;         // [2][BLK][VS]

  // tile order: (b, kv head, head within group, query block); blocks reading the same K/V
  // are consecutive and land on one XCD
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
  const int64_t qrs = (int64_t)Hq * D;         // token stride of q/out
  const int64_t krs = (int64_t)Hkv * D;        // token stride of k/v

  // Q^T as B operand: lane holds q[row = 32*wave + l32][d = 16s + 8*half .. +7]
  const int64_t qrow = (int64_t)b * N + (int64_t)i * BLK + 32 * wave + l32;
  bf16x8 qf[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(q + qrow * qrs + (int64_t)h * D + 16 * s + 8 * half));

  const int32_t* myidx = idx + (((int64_t)b * Hq + h) * nb + i) * topk;
  const uint16_t* kbase0 = k + (int64_t)b * N * krs + (int64_t)g * D;
  const uint16_t* vbase0 = v + (int64_t)b * N * krs + (int64_t)g * D;

  // staging: thread owns 16-byte chunks ch = tid + NT*x of the tile, row ch/(D/8); the
  // per-lane element offsets inside a tile are fixed, only the (uniform) tile base moves
  u32x4 kreg[C::CH], vreg[C::CH];
  uint32_t goff[C::CH];                        // byte offsets (tile < 2^32 bytes)
#pragma unroll
  for (int x = 0; x < C::CH; ++x) {
    const int ch = tid + C::NT * x;
    goff[x] = (uint32_t)(((ch / (D / 8)) * krs + (ch % (D / 8)) * 8) * 2);
  }
  bool bad = false;
  auto load_tile = [&](int kb) {
    if ((unsigned)kb >= (unsigned)nb) { bad = true; kb = 0; }
    const char* kt = (const char*)(kbase0 + (int64_t)kb * BLK * krs);
    const char* vt = (const char*)(vbase0 + (int64_t)kb * BLK * krs);
#pragma unroll
    for (int x = 0; x < C::CH; ++x) {
      kreg[x] = *(const u32x4*)(kt + goff[x]);
      vreg[x] = *(const u32x4*)(vt + goff[x]);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int x = 0; x < C::CH; ++x) {
      const int ch = tid + C::NT * x;
      const int r = ch / (D / 8), dc = ch % (D / 8);
      *(u32x4*)(Ks + buf * C::K_ELEMS + r * C::KS + dc * 8) = kreg[x];
      *(u32x4*)(Vs + buf * C::V_ELEMS + r * C::VS + dc * 8) = vreg[x];
    }
  };

  // transpose-read address of this lane inside a V tile: in each 16-lane group the lane
  // 4e+t names row (key) 4*half + e and columns d0 + 4t, d0 = 16*((lane/16)&1)
  const int tr_off = (4 * half + ((lane & 15) >> 2)) * C::VS + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  f32x16 oacc[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float mc = 0.f;                              // c * reference max of this lane's query row
  float lsum = 0.f;                            // this lane's share of the normaliser
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  load_tile(myidx[0]);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < topk; ++t) {
    const int buf = t & 1;
    if (t + 1 < topk) load_tile(myidx[t + 1]);

    // S^T = K Q^T for this wave's 32 queries
    const uint16_t* ks = Ks + buf * C::K_ELEMS;
    f32x16 sacc[C::NKT];
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *(const u32x4*)(ks + (32 * kt + l32) * C::KS + 16 * s + 8 * half));
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kt], 0, 0, 0);
      }
    }

    auto row_max_c = [&]() {                   // c * max over this block of the lane's row
      float mt = sacc[0][0];
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kt][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      return mt * c;
    };
    if (t == 0) mc = row_max_c();

    // weights as packed bf16 pairs, grouped per PV k-step; per-lane block sum
    uint32_t pw[C::NPS][4];
    float bsum = 0.f;
    auto weights = [&]() {
      bsum = 0.f;
#pragma unroll
      for (int s = 0; s < C::NPS; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[s >> 1][8 * (s & 1) + 2 * e], c, -mc));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[s >> 1][8 * (s & 1) + 2 * e + 1], c, -mc));
          const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
          pw[s][e] = __builtin_bit_cast(uint32_t, pp);
          bsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, bsum, false);
        }
    };
    weights();
    if (__ballot(bsum > kRescaleSum)) {        // rare: move the reference max up
      const float m_new = fmaxf(mc, row_max_c());
      const float alpha = __builtin_amdgcn_exp2f(mc - m_new);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      mc = m_new;
      weights();
    }
    lsum += bsum;

    // O^T += V^T P^T
    const uint16_t* vs = Vs + buf * C::V_ELEMS + tr_off;
#pragma unroll
    for (int s = 0; s < C::NPS; ++s) {
      const u32x4 pv = {pw[s][0], pw[s][1], pw[s][2], pw[s][3]};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pv);
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        const s16x4 lo = ds_read_tr16(vs + (16 * s) * C::VS + 32 * dt);
        const s16x4 hi = ds_read_tr16(vs + (16 * s + 8) * C::VS + 32 * dt);
        const s16x4 a8[2] = {lo, hi};
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb,
                                                           oacc[dt], 0, 0, 0);
      }
    }

    if (t + 1 < topk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: O = O^T / l, bf16, 4 consecutive d per store
  const float l_all = lsum + __shfl_xor(lsum, 32);
  const float inv = bad ? __builtin_nanf("") : 1.0f / l_all;
  uint16_t* orow = out + qrow * qrs + (int64_t)h * D;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * dt + 8 * j + 4 * half;
      u32x2 w;
      w[0] = pack_bf16x2(oacc[dt][4 * j + 0] * inv, oacc[dt][4 * j + 1] * inv);
      w[1] = pack_bf16x2(oacc[dt][4 * j + 2] * inv, oacc[dt][4 * j + 3] * inv);
      *(u32x2*)(orow + d0) = w;
    }
}

template <int D, int BLK>
hipError_t launch(int64_t B, int64_t N, int Hq, int Hkv, int topk, const void* q, const void* k,
                  const void* v, const int32_t* idx, float c, void* out, hipStream_t stream) {
  const int nb = (int)(N / BLK);
  const uint32_t total = (uint32_t)(B * Hq * nb);
  attn_bf16_kernel<D, BLK><<<total, Cfg<D, BLK>::NT, 0, stream>>>(
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, idx, (uint16_t*)out, N, Hq,
      Hkv, nb, topk, c, total);
  return hipGetLastError();
}

}  // namespace

bool attn_bf16_supported(int D, int block) {
  return (D == 64 || D == 128) && (block == 64 || block == 128);
}

hipError_t launch_attn_bf16(int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                            const void* q, const void* k, const void* v, const int32_t* idx,
                            float scale, void* out, hipStream_t stream) {
  const float c = (float)((double)scale * 1.4426950408889634);   // scale * log2(e)
  if (D == 64 && block == 64) return launch<64, 64>(B, N, Hq, Hkv, topk, q, k, v, idx, c, out, stream);
  if (D == 64 && block == 128) return launch<64, 128>(B, N, Hq, Hkv, topk, q, k, v, idx, c, out, stream);
  if (D == 128 && block == 64) return launch<128, 64>(B, N, Hq, Hkv, topk, q, k, v, idx, c, out, stream);
  return launch<128, 128>(B, N, Hq, Hkv, topk, q, k, v, idx, c, out, stream);
}

}  // namespace bsattn
