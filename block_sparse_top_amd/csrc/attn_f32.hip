// Step 4 for fp32 inputs: attention over the gathered selected blocks on the fp32 ALUs.
//
// Same operation as the bf16 kernel (SparseFormer page "2026 新一代卷积与Transformer网络架构
// 技术演进与性能对比", "SparseFormer 注意力实现" step 3; MSA page "从M2.7到M3：多模态模型稀疏
// 注意力架构设计与实现全解析" §2.1 with a block mask) with every product, exponent and sum in
// fp32, for inputs whose precision must be kept (max-abs error ~1e-6 on N(0,1) data).
//
// One work-group per (batch, query head, query block), one thread per query row. Keys of a
// selected block are staged 32 at a time in LDS (K and V rows, read as broadcasts); each
// thread keeps its q row, output row, running max and normaliser in registers and updates
// them once per 32 keys (exact online softmax: rescale whenever the max grows).
//
// Causal variant (template flag): query block i reads the first min(topk, i+1) entries of its
// row, each in [0, i]; in its own block keys after the query score -inf (weight 0). The first
// chunk of the own block always holds key 0 <= query, so no chunk starts from an all -inf max.
// Overlapping key blocks (template flag; the MSA page's §5.3): block j's keys are read from
// key_tile_start and its first key_tile_skip keys score -inf (chunks wholly before them are
// not read, so every chunk read holds a key that counts).
#include "common.h"
#include "launch.h"

namespace bsattn {
namespace {

constexpr int kChunk = 32;

template <int D, bool CAUSAL, bool OVL>
__global__ __launch_bounds__(128) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ idx, float* __restrict__ out, float* __restrict__ lse,
    int64_t N, int Hq, int Hkv, int nb, int block, int topk, float c, uint32_t total_tiles,
    int nkb, int kstride) {
  __shared__ __attribute__((aligned(16))) float ks[kChunk][D];
  __shared__ __attribute__((aligned(16))) float vs[kChunk][D];
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
  const int tid = threadIdx.x;
  const int64_t qrs = (int64_t)Hq * D, krs = (int64_t)Hkv * D;

  const int64_t row = (int64_t)b * N + (int64_t)i * block + tid;
  float qr[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = q[row * qrs + (int64_t)h * D + d];
    o[d] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;
  bool bad = false;
  const int32_t* myidx = idx + (((int64_t)b * Hq + h) * nb + i) * topk;
  const float* kb0 = k + (int64_t)b * N * krs + (int64_t)g * D;
  const float* vb0 = v + (int64_t)b * N * krs + (int64_t)g * D;

  const int kcount = CAUSAL && i + 1 < topk ? i + 1 : topk;
  const unsigned klim = CAUSAL ? (unsigned)(i + 1) : (unsigned)(OVL ? nkb : nb);
  if (OVL) mark_selected(chosen, myidx, kcount, nkb, tid, block);
  for (int t = 0; t < kcount; ++t) {
    int kb = myidx[t];
    if ((unsigned)kb >= klim) { bad = true; kb = 0; }
    const bool own = CAUSAL && kb == i;
    const int64_t first = OVL ? key_tile_start(kb, kstride, block, N) : (int64_t)kb * block;
    const int skip = OVL ? key_tile_skip(kb, kstride, block, N, is_selected(chosen, kb - 1)) : 0;
    for (int c0 = skip & ~(kChunk - 1); c0 < block; c0 += kChunk) {
      __syncthreads();
      for (int e = tid; e < kChunk * D / 4; e += block) {
        const int r = e / (D / 4), d4 = e % (D / 4);
        const int64_t tok = first + c0 + r;
        *(f32x4*)&ks[r][4 * d4] = *(const f32x4*)(kb0 + tok * krs + 4 * d4);
        *(f32x4*)&vs[r][4 * d4] = *(const f32x4*)(vb0 + tok * krs + 4 * d4);
      }
      __syncthreads();
      float s[kChunk];
      float mc = m;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        float a = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) a = __builtin_fmaf(qr[d], ks[j][d], a);
        s[j] = a * c;                          // exp2 domain
        if (own && c0 + j > tid) s[j] = -__builtin_inff();
        if (OVL && c0 + j < skip) s[j] = -__builtin_inff();
        mc = fmaxf(mc, s[j]);
      }
      const float alpha = __builtin_amdgcn_exp2f(m - mc);   // 0 on the first chunk
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= alpha;
      m = mc;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const float p = __builtin_amdgcn_exp2f(s[j] - m);
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, vs[j][d], o[d]);
      }
    }
  }
  const float inv = bad ? __builtin_nanf("") : 1.0f / l;
  if (lse)                                     // natural log-sum-exp of the row's scaled scores
    lse[((int64_t)b * Hq + h) * N + (int64_t)i * block + tid] =
        bad ? __builtin_nanf("") : (m + log2f(l)) * 0.6931471805599453f;
#pragma unroll
  for (int d = 0; d < D; ++d) out[row * qrs + (int64_t)h * D + d] = o[d] * inv;
}

template <int D>
hipError_t launch(int64_t B, int64_t N, int Hq, int Hkv, int block, int topk, const void* q,
                  const void* k, const void* v, const int32_t* idx, float c, void* out,
                  float* lse, bool causal, int nkb, int kstride, hipStream_t stream) {
  const int nb = (int)(N / block);
  const uint32_t total = (uint32_t)(B * Hq * nb);
#define BSATTN_F32_LAUNCH(causal_, ovl_)                                                     \
  attn_f32_kernel<D, causal_, ovl_><<<total, block, 0, stream>>>(                             \
      (const float*)q, (const float*)k, (const float*)v, idx, (float*)out, lse, N, Hq, Hkv, nb, \
      block, topk, c, total, nkb, kstride)
  if (causal)
    BSATTN_F32_LAUNCH(true, false);
  else if (kstride != block)
    BSATTN_F32_LAUNCH(false, true);
  else
    BSATTN_F32_LAUNCH(false, false);
#undef BSATTN_F32_LAUNCH
  return hipGetLastError();
}

}  // namespace

bool attn_f32_supported(int D, int block) {
  return (D == 64 || D == 128) && (block == 64 || block == 128);
}

hipError_t launch_attn_f32(int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                           const void* q, const void* k, const void* v, const int32_t* idx,
                           float scale, void* out, float* lse, bool causal, int key_stride,
                           int64_t nkb, hipStream_t stream) {
  const float c = (float)((double)scale * 1.4426950408889634);   // scale * log2(e)
  if (D == 64)
    return launch<64>(B, N, Hq, Hkv, block, topk, q, k, v, idx, c, out, lse, causal, (int)nkb,
                      key_stride, stream);
  return launch<128>(B, N, Hq, Hkv, block, topk, q, k, v, idx, c, out, lse, causal, (int)nkb,
                     key_stride, stream);
}

}  // namespace bsattn
