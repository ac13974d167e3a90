// The (D = 64, block = 64) kernels of attn_bf16_kernel.h: the SparseFormer page's own shape
// ("SparseFormer 注意力实现": 64-token blocks; "基准测试": hidden 1024 over 16 heads). This
// translation unit is compiled with the iterative ILP machine scheduler (build.py): on that
// shape it placed the softmax between the MFMAs better than the default (0.6-0.7 % faster on
// two boxes, same outputs), while the D = 128 kernels were slower with it.
#include "attn_bf16_kernel.h"

namespace bsattn {

hipError_t launch_attn_bf16_d64b64(int64_t B, int64_t N, int Hq, int Hkv, int topk,
                                   const void* q, const void* k, const void* v,
                                   const int32_t* idx, float c, void* out, float* lse,
                                   bool causal, int nk, int key_stride, hipStream_t stream) {
  // plain and causal key blocks only (the overlapping-block kernel is launched from
  // attn_bf16.hip, which calls this with key_stride = 64)
  return launch_tiles<64, 64, 64, 64, false>(B, N, Hq, Hkv, topk, q, k, v, idx, c, out, lse,
                                             causal, nk, key_stride, stream);
}

}  // namespace bsattn
