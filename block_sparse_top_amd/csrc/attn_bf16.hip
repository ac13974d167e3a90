// Step 4 for bf16 inputs: the launch side of the kernel in attn_bf16_kernel.h (SparseFormer
// page, "SparseFormer 注意力实现" step 3; MSA page §2.1, §2.2, §3.1). The (D = 64, block = 64)
// kernels, the SparseFormer page's own shape, are built in attn_bf16_page.hip.
#include "attn_bf16_kernel.h"

namespace bsattn {

bool attn_bf16_supported(int D, int block) {
  return (D == 64 || D == 128) && (block == 64 || block == 128);
}

hipError_t launch_attn_bf16(int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                            const void* q, const void* k, const void* v, const int32_t* idx,
                            float scale, void* out, float* lse, bool causal, int key_stride,
                            int64_t nkb, hipStream_t stream) {
  const float c = (float)((double)scale * 1.4426950408889634);   // scale * log2(e)
  const int nk = (int)nkb;
  // plain and causal: attn_bf16_page.hip; overlapping key blocks stay here (under the other
  // scheduler that kernel would need more than 256 registers)
  if (D == 64 && block == 64 && key_stride == block)
    return launch_attn_bf16_d64b64(B, N, Hq, Hkv, topk, q, k, v, idx, c, out, lse, causal, nk,
                                   key_stride, stream);
#define BSATTN_BF16_SHAPE(d_, b_) \
  launch<d_, b_>(B, N, Hq, Hkv, topk, q, k, v, idx, c, out, lse, causal, nk, key_stride, stream)
  if (D == 64 && block == 64) return BSATTN_BF16_SHAPE(64, 64);
  if (D == 64 && block == 128) return BSATTN_BF16_SHAPE(64, 128);
  if (D == 128 && block == 64) return BSATTN_BF16_SHAPE(128, 64);
  return BSATTN_BF16_SHAPE(128, 128);
#undef BSATTN_BF16_SHAPE
}

}  // namespace bsattn
