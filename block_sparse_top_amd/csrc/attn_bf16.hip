// Step 4: attention over the gathered selected blocks, bf16 inputs, bf16 MFMA (gfx950).
//
// SparseFormer page ("2026 新一代卷积与Transformer网络架构技术演进与性能对比"), section
// "SparseFormer 注意力实现", step 3: attention is computed only over the selected blocks with
// scale 1/sqrt(D); MSA page ("从M2.7到M3：多模态模型稀疏注意力架构设计与实现全解析") §2.1:
// Softmax(Mask(Q K^T / sqrt(d_k))) V with a block mask, §2.2: full attention inside the chosen
// blocks, §3.1: GQA. The softmax is exact: it is evaluated online over the k selected key
// blocks with a running maximum and normaliser in fp32.
//
// One work-group owns one query block (BLK rows) of one (batch, query head); each of its
// BLK/32 waves owns 32 query rows. Per selected key block the work-group stages K [BLK][D]
// row-major and V transposed [D][BLK] in LDS (two buffers: the next block's global loads are
// issued before the current block's math), then each wave computes
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = its Q^T in registers)
//   P^T = exp2(c*S^T - c*m)   (c = scale*log2(e), m = running row max)
//   O^T += V^T P^T (A = V^T rows from LDS, B = P^T straight from the S^T accumulators)
// Working on the transposed products keeps every query's 64 key scores in two lanes (l and
// l^32): the row max needs one cross-lane exchange, the rescale factor is one value per lane,
// and the score accumulators are already in the B-operand layout of the next product (the
// 16 k-slots of a step are matched to keys {4h..4h+3, 8+4h..8+4h+3} on both operands).
// The running max is only moved when a block's max exceeds it by more than 2^8 in the
// exp2 domain, so the O rescale is skipped for almost every block; the final O/l is exact
// either way because O and l always use the same reference maximum.
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

constexpr float kLazyRescaleLog2 = 8.0f;

template <int D, int BLK>
struct Cfg {
  static constexpr int NW = BLK / 32;          // waves (32 query rows each)
  static constexpr int NT = NW * kWave;        // threads
  static constexpr int KS = D + 8;             // K row stride in LDS (bf16 elements)
  static constexpr int VS = BLK + 4;           // V^T row stride in LDS (bf16 elements)
  static constexpr int K_ELEMS = BLK * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int LDS_BYTES = 2 * (K_ELEMS + V_ELEMS) * 2;
  static constexpr int KCH = D / 16;           // 16-byte K chunks per thread per block
  static constexpr int VU = D / 32;            // V units (2 rows x 16 bytes) per thread
  static constexpr int NKT = BLK / 32;         // 32-key sub-tiles per block
  static constexpr int NS = D / 16;            // k-steps of Q K^T
  static constexpr int NDT = D / 32;           // 32-row d tiles of O^T
  static constexpr int NPS = BLK / 16;         // k-steps of V^T P^T
};

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, uint16_t* __restrict__ out,
    int64_t N, int Hq, int Hkv, int nb, int topk, float c, uint32_t total_tiles) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (C::K_ELEMS + C::V_ELEMS)];
  uint16_t* Ks = lds;                          // [2][BLK][KS]
  uint16_t* Vt = lds + 2 * C::K_ELEMS;         // [2][D][VS]

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

  u32x4 kreg[C::KCH];
  u32x4 vreg[C::VU][2];
  bool bad = false;

  auto load_tile = [&](int kb) {
    if ((unsigned)kb >= (unsigned)nb) { bad = true; kb = 0; }
    const uint16_t* kb_ptr = kbase0 + (int64_t)kb * BLK * krs;
    const uint16_t* vb_ptr = vbase0 + (int64_t)kb * BLK * krs;
#pragma unroll
    for (int x = 0; x < C::KCH; ++x) {
      const int ch = tid + C::NT * x;
      const int r = ch / (D / 8), dc = ch % (D / 8);
      kreg[x] = *(const u32x4*)(kb_ptr + r * krs + dc * 8);
    }
#pragma unroll
    for (int x = 0; x < C::VU; ++x) {
      const int u = tid + C::NT * x;
      const int m = u % (BLK / 2), dc = u / (BLK / 2);
      vreg[x][0] = *(const u32x4*)(vb_ptr + (2 * m) * krs + dc * 8);
      vreg[x][1] = *(const u32x4*)(vb_ptr + (2 * m + 1) * krs + dc * 8);
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks = Ks + buf * C::K_ELEMS;
    uint32_t* vt = (uint32_t*)(Vt + buf * C::V_ELEMS);
#pragma unroll
    for (int x = 0; x < C::KCH; ++x) {
      const int ch = tid + C::NT * x;
      const int r = ch / (D / 8), dc = ch % (D / 8);
      *(u32x4*)(ks + r * C::KS + dc * 8) = kreg[x];
    }
#pragma unroll
    for (int x = 0; x < C::VU; ++x) {
      const int u = tid + C::NT * x;
      const int m = u % (BLK / 2), dc = u / (BLK / 2);
      const u32x4 a = vreg[x][0], bb = vreg[x][1];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // (v[2m][d], v[2m+1][d]) for d = 8dc + 2w and 8dc + 2w + 1
        const uint32_t lo = __builtin_amdgcn_perm(bb[w], a[w], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(bb[w], a[w], 0x07060302u);
        vt[(dc * 8 + 2 * w) * (C::VS / 2) + m] = lo;
        vt[(dc * 8 + 2 * w + 1) * (C::VS / 2) + m] = hi;
      }
    }
  };

  f32x16 oacc[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_used = -__builtin_inff();            // reference max of this lane's query row
  float lsum = 0.f;                            // this lane's share of the normaliser

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

    // online softmax (lane pair l, l^32 shares one query row)
    float mt = sacc[0][0];
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kt][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool grow = (mt - m_used) * c > kLazyRescaleLog2;
    if (__ballot(grow)) {
      const float m_new = fmaxf(m_used, mt);
      const float alpha = __builtin_amdgcn_exp2f((m_used - m_new) * c);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m_used = m_new;
    }
    const float mc = m_used * c;
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r], c, -mc));
        lsum += p;
        sacc[kt][r] = p;
      }

    // O^T += V^T P^T
    const uint16_t* vt = Vt + buf * C::V_ELEMS;
#pragma unroll
    for (int s = 0; s < C::NPS; ++s) {
      const f32x16& pa = sacc[s >> 1];
      const int o8 = 8 * (s & 1);
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)pa[o8 + e];
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        const uint16_t* row = vt + (32 * dt + l32) * C::VS + 16 * s + 4 * half;
        const u32x2 lo = *(const u32x2*)(row);
        const u32x2 hi = *(const u32x2*)(row + 8);
        const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb,
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
