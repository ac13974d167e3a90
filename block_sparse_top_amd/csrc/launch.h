// Internal launchers of the gfx950 kernels. Shapes are validated by the C ABI layer
// before any of these is called; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsattn {

// Step 1: per-block mean (fp32 out, [B, H, nblk, D]) of the tensors in `which` (bit 0: q,
// bit 1: k). kind: 0 fp32, 1 bf16, 2 fp8. q has nb = N / block blocks; k has nkb key blocks
// starting every key_stride tokens (key_stride == block: the same nb blocks).
hipError_t launch_pool(int kind, int which, int64_t B, int64_t N, int Hq, int Hkv, int D,
                       int block, int key_stride, int64_t nkb, const void* q, const void* k,
                       float* qbar, float* kbar, bool pmax, hipStream_t stream);

// Steps 1 (query side), 2 and 3 fused for nkb <= kMaxFusedBlocks key blocks: query pooling
// (also stored to qbar), block scores against the nkb pooled keys kbar, top-k per row.
constexpr int kMaxFusedBlocks = 1024;
hipError_t launch_pool_score_select(int kind, int64_t B, int64_t N, int Hq, int Hkv, int D,
                                    int block, int topk, int64_t nkb, const void* q, float* qbar,
                                    const float* kbar, int32_t* idx, unsigned flags,
                                    int nrand, uint64_t seed, hipStream_t stream);

// Steps 2-3 for nb > kMaxFusedBlocks (nb % 64 == 0, nb <= kMaxLargeBlocks): S = scores
// [B, Hq, nb, nb] fp32 in the workspace ([B, Hkv, nb, nb] with group), then the top-k of each
// of its rows.
constexpr int kMaxLargeBlocks = 8192;

// Whether a selection over nb key blocks writes the score matrix to the workspace (measured:
// at nb = 1024 the fused kernel is faster than the score matrix path, 2.1 ms against 3.0 ms
// for the 64K-token fp8 workload, so the fused kernel serves every nb up to 1024).
inline bool materialized_scores(int64_t nb, bool group) {
  (void)group;
  return nb > kMaxFusedBlocks;
}
// group: the pooled queries of each KV group are summed in place into the rows of its first
// head and S holds one [nb, nb] matrix per (batch, KV head); topk_rows then writes each row to
// the idx rows of the G heads of its group (G = 1: one row each). causal: only the tiles on and
// below the diagonal of each matrix are formed (the causal top-k reads no others).
hipError_t launch_scores_large(int64_t B, int Hq, int Hkv, int nb, int D, float* qbar,
                               const float* kbar, float* S, bool group, bool causal,
                               hipStream_t stream);
hipError_t launch_topk_rows(int64_t rows, int nb, int topk, const float* S, int32_t* idx,
                            bool causal, int G, hipStream_t stream);

// Overlapping key blocks: at most this many per sequence in attention (an LDS bitmap of a
// row's chosen blocks); the selection takes up to kMaxFusedBlocks of them.
constexpr int kMaxKeyBlocks = 8192;

// Step 4, bf16 inputs on bf16 MFMA. Supported (D, block): D, block in {64, 128}.
// key_stride == block: plain key blocks; otherwise nkb overlapping key blocks (not causal).
bool attn_bf16_supported(int D, int block);
hipError_t launch_attn_bf16(int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                            const void* q, const void* k, const void* v, const int32_t* idx,
                            float scale, void* out, float* lse, bool causal, int key_stride,
                            int64_t nkb, hipStream_t stream);
// the (D = 64, block = 64) kernels of launch_attn_bf16, built in their own translation unit
// (attn_bf16_page.hip); c = scale * log2(e), nk key blocks
hipError_t launch_attn_bf16_d64b64(int64_t B, int64_t N, int Hq, int Hkv, int topk,
                                   const void* q, const void* k, const void* v,
                                   const int32_t* idx, float c, void* out, float* lse,
                                   bool causal, int nk, int key_stride, hipStream_t stream);

// Step 4, fp32 inputs on the fp32 vector ALUs (key blocks as for bf16).
bool attn_f32_supported(int D, int block);
hipError_t launch_attn_f32(int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                           const void* q, const void* k, const void* v, const int32_t* idx,
                           float scale, void* out, float* lse, bool causal, int key_stride,
                           int64_t nkb, hipStream_t stream);

// Step 4, OCP fp8 e4m3 inputs on the fp8 MFMA, bf16 output. Supported: D = 128,
// block in {64, 128}. descale_qkv: host array of the three per-tensor descales.
bool attn_fp8_supported(int D, int block);
hipError_t launch_attn_fp8(int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                           const void* q, const void* k, const void* v, const int32_t* idx,
                           float scale, const float* descale_qkv, void* out, float* lse,
                           bool causal, int key_stride, int64_t nkb, hipStream_t stream);

// Backward (bf16 inputs, fp32 gradients): supported for block 64 and 128, D in {64, 128}.
// dtype_kind: 0 fp32, 1 bf16, 2 fp8. Workspace: Dvec [B,Hq,N] fp32, key-block offsets
// [B,Hkv,nb+1], pair lists [B,Hq,nb,topk] int32 (block 128: those of the 64-token form with
// 2*topk places, then its index rows [B,Hq,N/64,2*topk] written by launch_expand_idx128).
// launch_attn_bwd works on 64-token blocks.
constexpr int kMaxBwdBlocks = 4096;
bool attn_bwd_supported(int dtype_kind, int D, int block);
size_t attn_bwd_workspace_bytes(int64_t B, int64_t N, int Hq, int Hkv, int block, int topk);
hipError_t launch_expand_idx128(int64_t rows, int nb, int topk, bool causal, const int32_t* idx,
                                int32_t* idx64, hipStream_t stream);
hipError_t launch_attn_bwd(int64_t B, int64_t N, int Hq, int Hkv, int D, int topk, bool causal,
                           const void* q, const void* k, const void* v, const int32_t* idx,
                           const void* out, const void* dout, const float* lse, float scale,
                           float* dq, float* dk, float* dv, void* workspace,
                           hipStream_t stream);

// Decode step (bf16 caches; D in {64, 128}, block in {64, 128}, Lmax / block <= 8192).
int decode_splits(int64_t B, int Hq, int topk);
size_t decode_workspace_bytes(int64_t B, int Hq, int D, int topk);
bool decode_supported(int D, int block);
constexpr int kMaxDecodeBlocks = 8192;
hipError_t launch_decode_pool(int64_t B, int64_t Lmax, int Hkv, int D, int block,
                              const void* k_cache, const int32_t* lens_old,
                              const int32_t* lens_new, float* kbar, hipStream_t stream);
hipError_t launch_decode(int64_t B, int64_t Lmax, int Hq, int Hkv, int D, int block, int topk,
                         bool group, const void* q, const void* k_cache, const void* v_cache,
                         const float* kbar, const int32_t* lens, float scale, void* out,
                         int32_t* idx, void* workspace, hipStream_t stream);

// Checks every idx row (topk values, strictly ascending, in [0, nkb); causal: the first
// min(topk, i+1) values strictly ascending in [0, i] for query block i = row mod nb, the rest
// -1); waits for the stream and returns the number of failing rows in *bad_rows. counter:
// 4 bytes of device memory the call may overwrite (zeroed first, then counted into).
hipError_t validate_idx(int64_t rows, int topk, int nb, int nkb, const int32_t* idx,
                        bool causal, unsigned int* counter, hipStream_t stream,
                        unsigned int* bad_rows);

}  // namespace bsattn
