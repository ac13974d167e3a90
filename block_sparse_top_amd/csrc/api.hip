// C ABI of the library (declared in include/bsattn.h): host-side argument checks,
// workspace layout, and dispatch of the gfx950 kernels onto the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/bsattn.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BSATTN_OK;
  return fail(BSATTN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// BSATTN_VALIDATE=1 in the environment: bsattn_forward checks idx on the GPU first
bool validate_enabled() {
  const char* v = getenv("BSATTN_VALIDATE");
  return v && v[0] == '1' && v[1] == 0;
}

// Key blocks of a sequence of N tokens (N % block == 0) at the key stride ks (block: the nb
// blocks of the partition; below: overlapping blocks, the last one ending at token N).
int64_t key_count(int64_t N, int block, int ks) {
  if (N == 0) return 0;
  if (ks == block) return N / block;
  return (N - block + ks - 1) / ks + 1;
}

// Shape checks common to the entry points. key_stride 0 means block. Returns BSATTN_OK or an
// error with detail.
int check_shape(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                int key_stride) {
  if (dtype != BSATTN_F32 && dtype != BSATTN_BF16 && dtype != BSATTN_FP8_E4M3)
    return fail(BSATTN_E_INVALID, "unknown dtype %d", dtype);
  if (B < 0 || N < 0) return fail(BSATTN_E_INVALID, "negative B or N");
  if (Hq < 1 || Hkv < 1) return fail(BSATTN_E_INVALID, "Hq and Hkv must be >= 1");
  if (Hq % Hkv) return fail(BSATTN_E_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (D < 1 || block < 1) return fail(BSATTN_E_INVALID, "D and block must be >= 1");
  if (N % block) return fail(BSATTN_E_INVALID, "N (%lld) must be a multiple of block (%d)",
                             (long long)N, block);
  const int64_t nb = N / block;
  const int ks = key_stride == 0 ? block : key_stride;
  if (ks > block || 2 * (int64_t)ks < block)
    return fail(BSATTN_E_INVALID, "key_stride %d outside [block/2, block] (block=%d)", key_stride,
                block);
  const int64_t nkb = key_count(N, block, ks);
  if (B == 0 || N == 0) {
    if (topk < 0 || topk > nkb)
      return fail(BSATTN_E_INVALID, "topk %d outside [0, key blocks=%lld]", topk, (long long)nkb);
  } else if (topk < 1 || topk > nkb) {
    return fail(BSATTN_E_INVALID, "topk %d outside [1, key blocks=%lld]", topk, (long long)nkb);
  }
  if (D != 64 && D != 128) return fail(BSATTN_E_UNSUPPORTED, "D=%d (supported: 64, 128)", D);
  if (block != 64 && block != 128)
    return fail(BSATTN_E_UNSUPPORTED, "block=%d (supported: 64, 128)", block);
  // index arithmetic limits of the kernels: tiles and rows fit in 32 bits
  if (B * (int64_t)Hq * nb >= ((int64_t)1 << 31))
    return fail(BSATTN_E_UNSUPPORTED, "B*Hq*nb too large");
  if (N > ((int64_t)1 << 40)) return fail(BSATTN_E_UNSUPPORTED, "N too large");
  return BSATTN_OK;
}

size_t pooled_q_bytes(int64_t B, int64_t N, int Hq, int D, int block) {
  return align256((size_t)B * Hq * (size_t)(N / block) * D * sizeof(float));
}
size_t pooled_k_bytes(int64_t B, int64_t nkb, int Hkv, int D) {
  return align256((size_t)B * Hkv * (size_t)nkb * D * sizeof(float));
}
// score matrix, only for the many-block path
size_t scores_bytes(int64_t B, int64_t N, int Hq, int block) {
  const size_t nb = (size_t)(N / block);
  // the workspace query has no flags: size for the ungrouped selection (the larger one)
  if (!bsattn::materialized_scores((int64_t)nb, false)) return 0;
  return align256((size_t)B * Hq * nb * nb * sizeof(float));
}

}  // namespace

// ---- device scratch of bsattn_select_noalloc: a file-scope array of fixed size on every GPU
// the library runs on, held until the process ends. Host code never passes `scratch` itself
// (its host-side name is no device address): the address comes from hipGetSymbolAddress,
// once per device, and is kept in g_scratch_ptr.
namespace bsattn {
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];
}  // namespace bsattn

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the scratch array on the current device (looked up on first use there).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BSATTN_E_UNSUPPORTED, "device %d (the static scratch serves devices 0..%d)", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(bsattn::scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p & 255u))
      return fail(BSATTN_E_HIP, "scratch address %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BSATTN_OK;
}
}  // namespace

extern "C" {

int bsattn_abi_version(void) { return BSATTN_ABI_VERSION; }

size_t bsattn_select_noalloc_max_bytes(void) { return bsattn::kNoAllocScratchBytes; }

int bsattn_select_noalloc(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block,
                          int topk, unsigned flags, int nrand, uint64_t seed, int key_stride,
                          const void* q, const void* k, int32_t* idx, void* stream) {
  int st = check_shape(dtype, B, N, Hq, Hkv, D, block, topk, key_stride);
  if (st != BSATTN_OK) return st;
  const size_t need = bsattn_select_workspace_bytes_ex(B, N, Hq, Hkv, D, block, key_stride);
  if (need > bsattn::kNoAllocScratchBytes)
    return fail(BSATTN_E_WORKSPACE,
                "selection needs %zu bytes of scratch, the static scratch holds %zu "
                "(use bsattn_select_ex with a workspace)",
                need, bsattn::kNoAllocScratchBytes);
  if (B == 0 || N == 0)
    return bsattn_select_ex(dtype, B, N, Hq, Hkv, D, block, topk, flags, nrand, seed, key_stride,
                            q, k, idx, nullptr, 0, stream);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != BSATTN_OK) return st;
  return bsattn_select_ex(dtype, B, N, Hq, Hkv, D, block, topk, flags, nrand, seed, key_stride,
                          q, k, idx, ws, bsattn::kNoAllocScratchBytes, stream);
}

const char* bsattn_status_str(int status) {
  switch (status) {
    case BSATTN_OK: return "ok";
    case BSATTN_E_INVALID: return "invalid argument";
    case BSATTN_E_UNSUPPORTED: return "unsupported size or dtype";
    case BSATTN_E_WORKSPACE: return "workspace missing or too small";
    case BSATTN_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* bsattn_last_error(void) { return g_err; }

int64_t bsattn_key_blocks(int64_t N, int block, int key_stride) {
  if (N < 0 || block < 1 || N % block) {
    fail(BSATTN_E_INVALID, "N (%lld) must be >= 0 and a multiple of block (%d)", (long long)N,
         block);
    return -1;
  }
  const int ks = key_stride == 0 ? block : key_stride;
  if (ks > block || 2 * (int64_t)ks < block) {
    fail(BSATTN_E_INVALID, "key_stride %d outside [block/2, block] (block=%d)", key_stride, block);
    return -1;
  }
  return key_count(N, block, ks);
}

size_t bsattn_select_workspace_bytes_ex(int64_t B, int64_t N, int Hq, int Hkv, int D, int block,
                                        int key_stride) {
  if (B < 0 || N < 0 || Hq < 1 || Hkv < 1 || D < 1 || block < 1 || N % block) {
    fail(BSATTN_E_INVALID, "invalid sizes for the workspace query");
    return 0;
  }
  const int64_t nkb = bsattn_key_blocks(N, block, key_stride);
  if (nkb < 0) return 0;
  if (B == 0 || N == 0) return 0;
  return pooled_q_bytes(B, N, Hq, D, block) + pooled_k_bytes(B, nkb, Hkv, D) +
         scores_bytes(B, N, Hq, block);
}

size_t bsattn_select_workspace_bytes(int64_t B, int64_t N, int Hq, int Hkv, int D, int block) {
  return bsattn_select_workspace_bytes_ex(B, N, Hq, Hkv, D, block, 0);
}

int bsattn_select(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                  const void* q, const void* k, int32_t* idx, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return bsattn_select_ex(dtype, B, N, Hq, Hkv, D, block, topk, 0u, 0, 0ull, 0, q, k, idx,
                          workspace, workspace_bytes, stream);
}

int bsattn_select_ex(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block,
                     int topk, unsigned flags, int nrand, uint64_t seed, int key_stride,
                     const void* q, const void* k, int32_t* idx, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_shape(dtype, B, N, Hq, Hkv, D, block, topk, key_stride);
  if (st != BSATTN_OK) return st;
  const int ks = key_stride == 0 ? block : key_stride;
  const bool overlap = ks != block;
  if (flags & ~(unsigned)(BSATTN_CAUSAL | BSATTN_POOL_MAX | BSATTN_GROUP_SELECT))
    return fail(BSATTN_E_INVALID, "unknown flags 0x%x", flags);
  if (nrand < 0 || nrand > topk)
    return fail(BSATTN_E_INVALID, "nrand %d outside [0, topk=%d]", nrand, topk);
  if (nrand > 0 && (flags & BSATTN_CAUSAL))
    return fail(BSATTN_E_UNSUPPORTED, "random places with the causal selection");
  if (overlap && (flags & BSATTN_CAUSAL))
    return fail(BSATTN_E_UNSUPPORTED, "overlapping key blocks with the causal selection");
  if (B == 0 || N == 0) return BSATTN_OK;
  const int64_t nb = N / block;
  const int64_t nkb = key_count(N, block, ks);
  if (overlap && nkb > bsattn::kMaxFusedBlocks)
    return fail(BSATTN_E_UNSUPPORTED, "selection over %lld overlapping key blocks (supported: <= %d)",
                (long long)nkb, bsattn::kMaxFusedBlocks);
  const bool large = bsattn::materialized_scores(nb, flags & BSATTN_GROUP_SELECT);
  if (large && (nb > bsattn::kMaxLargeBlocks || nb % 64))
    return fail(BSATTN_E_UNSUPPORTED,
                "selection over nb=%lld blocks (supported: nb <= %d, or a multiple of 64 up to %d)",
                (long long)nb, bsattn::kMaxFusedBlocks, bsattn::kMaxLargeBlocks);
  if (large && nrand > 0)
    return fail(BSATTN_E_UNSUPPORTED, "random places over nb=%lld > %d blocks", (long long)nb,
                bsattn::kMaxFusedBlocks);
  if (!q || !k || !idx) return fail(BSATTN_E_INVALID, "null q, k or idx");
  if (!aligned16(q) || !aligned16(k) || ((uintptr_t)idx & 3u))
    return fail(BSATTN_E_INVALID, "q and k must be 16-byte aligned, idx 4-byte aligned");
  const size_t need = bsattn_select_workspace_bytes_ex(B, N, Hq, Hkv, D, block, key_stride);
  if (!workspace || workspace_bytes < need)
    return fail(BSATTN_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if ((uintptr_t)workspace & 255u) return fail(BSATTN_E_WORKSPACE, "workspace not 256-byte aligned");

  float* qbar = (float*)workspace;
  float* kbar = (float*)((char*)workspace + pooled_q_bytes(B, N, Hq, D, block));
  hipStream_t s = (hipStream_t)stream;
  const int kind = dtype == BSATTN_F32 ? 0 : dtype == BSATTN_BF16 ? 1 : 2;
  const bool pmax = flags & BSATTN_POOL_MAX, causal = flags & BSATTN_CAUSAL;
  if (large) {
    float* S = (float*)((char*)kbar + pooled_k_bytes(B, nkb, Hkv, D));
    st = hip_status(bsattn::launch_pool(kind, 3, B, N, Hq, Hkv, D, block, ks, nkb, q, k, qbar,
                                        kbar, pmax, s),
                    "pool launch");
    if (st != BSATTN_OK) return st;
    const bool group = flags & BSATTN_GROUP_SELECT;
    st = hip_status(bsattn::launch_scores_large(B, Hq, Hkv, (int)nb, D, qbar, kbar, S, group,
                                                causal, s),
                    "score launch");
    if (st != BSATTN_OK) return st;
    return hip_status(bsattn::launch_topk_rows(B * (group ? Hkv : Hq) * nb, (int)nb, topk, S, idx,
                                               causal, group ? Hq / Hkv : 1, s),
                      "top-k launch");
  }
  st = hip_status(bsattn::launch_pool(kind, 2, B, N, Hq, Hkv, D, block, ks, nkb, q, k, qbar,
                                      kbar, pmax, s),
                  "key pool launch");
  if (st != BSATTN_OK) return st;
  return hip_status(bsattn::launch_pool_score_select(kind, B, N, Hq, Hkv, D, block, topk, nkb,
                                                     q, qbar, kbar, idx, flags, nrand, seed, s),
                    "query pool/score/select launch");
}

int bsattn_forward(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                   const void* q, const void* k, const void* v, const int32_t* idx, float scale,
                   const float* descale_qkv, void* out, void* stream) {
  return bsattn_forward_ex(dtype, B, N, Hq, Hkv, D, block, topk, 0u, 0, q, k, v, idx, scale,
                           descale_qkv, out, nullptr, stream);
}

int bsattn_forward_ex(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block,
                      int topk, unsigned flags, int key_stride, const void* q, const void* k,
                      const void* v, const int32_t* idx, float scale, const float* descale_qkv,
                      void* out, float* lse, void* stream) {
  int st = check_shape(dtype, B, N, Hq, Hkv, D, block, topk, key_stride);
  if (st != BSATTN_OK) return st;
  if (flags & ~(unsigned)(BSATTN_CAUSAL | BSATTN_POOL_MAX | BSATTN_GROUP_SELECT))
    return fail(BSATTN_E_INVALID, "unknown flags 0x%x", flags);
  const bool causal = flags & BSATTN_CAUSAL;
  const int ks = key_stride == 0 ? block : key_stride;
  const int64_t nkb = key_count(N, block, ks);
  if (ks != block && causal)
    return fail(BSATTN_E_UNSUPPORTED, "overlapping key blocks with the causal variant");
  if (ks != block && nkb > bsattn::kMaxKeyBlocks)
    return fail(BSATTN_E_UNSUPPORTED, "attention over %lld overlapping key blocks (supported: <= %d)",
                (long long)nkb, bsattn::kMaxKeyBlocks);
  if (!isfinite(scale) || !(scale > 0.f))
    return fail(BSATTN_E_INVALID, "scale must be finite and > 0");
  if (dtype == BSATTN_FP8_E4M3) {
    if (!descale_qkv) return fail(BSATTN_E_INVALID, "fp8 needs descale_qkv");
    for (int j = 0; j < 3; ++j)
      if (!isfinite(descale_qkv[j]) || !(descale_qkv[j] > 0.f))
        return fail(BSATTN_E_INVALID, "descale_qkv[%d] must be finite and > 0", j);
  }
  if (B == 0 || N == 0) return BSATTN_OK;
  if (!q || !k || !v || !idx || !out) return fail(BSATTN_E_INVALID, "null pointer argument");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || ((uintptr_t)idx & 3u) ||
      ((uintptr_t)lse & 3u))
    return fail(BSATTN_E_INVALID,
                "q, k, v, out must be 16-byte aligned, idx and lse 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (validate_enabled()) {
    unsigned int bad = 0;
    const int64_t nb = N / block;
    st = hip_status(
        // the counter goes to the first 4 bytes of out, which the attention overwrites
        bsattn::validate_idx(B * Hq * nb, topk, (int)nb, (int)nkb, idx, causal,
                             (unsigned int*)out, s, &bad),
        "idx validation");
    if (st != BSATTN_OK) return st;
    if (bad)
      return fail(BSATTN_E_INVALID,
                  causal ? "idx: %u rows are not causal rows (strictly ascending in [0, i], "
                           "then -1; nb=%lld)"
                         : "idx: %u rows are not strictly ascending in [0, key blocks=%lld)",
                  bad, (long long)(causal ? nb : nkb));
  }
  if (dtype == BSATTN_BF16) {
    if (!bsattn::attn_bf16_supported(D, block))
      return fail(BSATTN_E_UNSUPPORTED, "bf16 attention for D=%d block=%d", D, block);
    return hip_status(bsattn::launch_attn_bf16(B, N, Hq, Hkv, D, block, topk, q, k, v, idx,
                                               scale, out, lse, causal, ks, nkb, s),
                      "bf16 attention launch");
  }
  if (dtype == BSATTN_F32) {
    if (!bsattn::attn_f32_supported(D, block))
      return fail(BSATTN_E_UNSUPPORTED, "fp32 attention for D=%d block=%d", D, block);
    return hip_status(bsattn::launch_attn_f32(B, N, Hq, Hkv, D, block, topk, q, k, v, idx,
                                              scale, out, lse, causal, ks, nkb, s),
                      "fp32 attention launch");
  }
  if (!bsattn::attn_fp8_supported(D, block))
    return fail(BSATTN_E_UNSUPPORTED, "fp8 attention for D=%d block=%d (supported: D=128)", D,
                block);
  return hip_status(bsattn::launch_attn_fp8(B, N, Hq, Hkv, D, block, topk, q, k, v, idx, scale,
                                            descale_qkv, out, lse, causal, ks, nkb, s),
                    "fp8 attention launch");
}

size_t bsattn_backward_workspace_bytes(int64_t B, int64_t N, int Hq, int Hkv, int D, int block,
                                       int topk) {
  (void)D;
  if (B < 0 || N < 0 || Hq < 1 || Hkv < 1 || block < 1 || N % block || topk < 0) {
    fail(BSATTN_E_INVALID, "invalid sizes for the workspace query");
    return 0;
  }
  if (B == 0 || N == 0) return 0;
  return bsattn::attn_bwd_workspace_bytes(B, N, Hq, Hkv, block, topk);
}

int bsattn_backward(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                    unsigned flags, const void* q, const void* k, const void* v,
                    const int32_t* idx, const void* out, const void* dout, const float* lse,
                    float scale, float* dq, float* dk, float* dv, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int st = check_shape(dtype, B, N, Hq, Hkv, D, block, topk, 0);
  if (st != BSATTN_OK) return st;
  if (flags & ~(unsigned)(BSATTN_CAUSAL | BSATTN_POOL_MAX | BSATTN_GROUP_SELECT))
    return fail(BSATTN_E_INVALID, "unknown flags 0x%x", flags);
  if (!isfinite(scale) || !(scale > 0.f))
    return fail(BSATTN_E_INVALID, "scale must be finite and > 0");
  const int kind = dtype == BSATTN_F32 ? 0 : dtype == BSATTN_BF16 ? 1 : 2;
  if (!bsattn::attn_bwd_supported(kind, D, block))
    return fail(BSATTN_E_UNSUPPORTED, "backward for dtype %d D=%d block=%d (supported: bf16, "
                                      "D 64 or 128, block 64 or 128)", dtype, D, block);
  if (N / 64 > bsattn::kMaxBwdBlocks)
    return fail(BSATTN_E_UNSUPPORTED, "backward over %lld 64-token blocks > %d",
                (long long)(N / 64), bsattn::kMaxBwdBlocks);
  if (B == 0 || N == 0) return BSATTN_OK;
  if (!q || !k || !v || !idx || !out || !dout || !lse || !dq || !dk || !dv)
    return fail(BSATTN_E_INVALID, "null pointer argument");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || ((uintptr_t)idx & 3u) ||
      ((uintptr_t)lse & 3u))
    return fail(BSATTN_E_INVALID, "tensors must be 16-byte aligned, idx and lse 4-byte aligned");
  const size_t need = bsattn::attn_bwd_workspace_bytes(B, N, Hq, Hkv, block, topk);
  if (!workspace || workspace_bytes < need)
    return fail(BSATTN_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if ((uintptr_t)workspace & 255u) return fail(BSATTN_E_WORKSPACE, "workspace not 256-byte aligned");
  const bool causal = flags & BSATTN_CAUSAL;
  hipStream_t s = (hipStream_t)stream;
  if (block == 128) {                         // as 64-token blocks with expanded index rows
    int32_t* idx64 = (int32_t*)((char*)workspace +
                                bsattn::attn_bwd_workspace_bytes(B, N, Hq, Hkv, 64, 2 * topk));
    st = hip_status(bsattn::launch_expand_idx128(B * Hq * (N / 128), (int)(N / 128), topk,
                                                 causal, idx, idx64, s),
                    "index expansion launch");
    if (st != BSATTN_OK) return st;
    return hip_status(bsattn::launch_attn_bwd(B, N, Hq, Hkv, D, 2 * topk, causal, q, k, v, idx64,
                                              out, dout, lse, scale, dq, dk, dv, workspace, s),
                      "backward launch");
  }
  return hip_status(bsattn::launch_attn_bwd(B, N, Hq, Hkv, D, topk, causal, q, k, v, idx, out,
                                            dout, lse, scale, dq, dk, dv, workspace, s),
                    "backward launch");
}

namespace {

// sizes shared by the decode entry points
int check_decode(int dtype, int64_t B, int64_t Lmax, int Hq, int Hkv, int D, int block) {
  if (dtype != BSATTN_F32 && dtype != BSATTN_BF16 && dtype != BSATTN_FP8_E4M3)
    return fail(BSATTN_E_INVALID, "unknown dtype %d", dtype);
  if (B < 0 || Lmax < 0) return fail(BSATTN_E_INVALID, "negative B or Lmax");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv)
    return fail(BSATTN_E_INVALID, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  if (block < 1 || Lmax % block)
    return fail(BSATTN_E_INVALID, "Lmax (%lld) must be a multiple of block (%d)",
                (long long)Lmax, block);
  if (dtype != BSATTN_BF16) return fail(BSATTN_E_UNSUPPORTED, "decode for dtype %d (bf16 only)", dtype);
  if (!bsattn::decode_supported(D, block))
    return fail(BSATTN_E_UNSUPPORTED, "decode for D=%d block=%d", D, block);
  if (Lmax / block > bsattn::kMaxDecodeBlocks)
    return fail(BSATTN_E_UNSUPPORTED, "decode over %lld > %d blocks", (long long)(Lmax / block),
                bsattn::kMaxDecodeBlocks);
  if (B > 65535) return fail(BSATTN_E_UNSUPPORTED, "decode batch B=%lld > 65535", (long long)B);
  if (B * (int64_t)Hq * 64 >= ((int64_t)1 << 31)) return fail(BSATTN_E_UNSUPPORTED, "B*Hq too large");
  return BSATTN_OK;
}

}  // namespace

size_t bsattn_decode_workspace_bytes(int64_t B, int Hq, int D, int topk) {
  if (B < 0 || Hq < 1 || D < 1 || topk < 1) {
    fail(BSATTN_E_INVALID, "invalid sizes for the workspace query");
    return 0;
  }
  if (B == 0) return 0;
  return bsattn::decode_workspace_bytes(B, Hq, D, topk);
}

int bsattn_decode_pool(int dtype, int64_t B, int64_t Lmax, int Hkv, int D, int block,
                       const void* k_cache, const int32_t* lens_old, const int32_t* lens_new,
                       float* kbar, void* stream) {
  int st = check_decode(dtype, B, Lmax, Hkv, Hkv, D, block);
  if (st != BSATTN_OK) return st;
  if (B == 0 || Lmax == 0) return BSATTN_OK;
  if (!k_cache || !lens_new || !kbar) return fail(BSATTN_E_INVALID, "null pointer argument");
  if (!aligned16(k_cache) || !aligned16(kbar) || ((uintptr_t)lens_new & 3u) ||
      ((uintptr_t)lens_old & 3u))
    return fail(BSATTN_E_INVALID, "k_cache and kbar must be 16-byte aligned, lens 4-byte aligned");
  return hip_status(bsattn::launch_decode_pool(B, Lmax, Hkv, D, block, k_cache, lens_old,
                                               lens_new, kbar, (hipStream_t)stream),
                    "decode pool launch");
}

int bsattn_decode(int dtype, int64_t B, int64_t Lmax, int Hq, int Hkv, int D, int block, int topk,
                  const void* q, const void* k_cache, const void* v_cache, const float* kbar,
                  const int32_t* lens, float scale, void* out, int32_t* idx, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return bsattn_decode_ex(dtype, B, Lmax, Hq, Hkv, D, block, topk, 0u, q, k_cache, v_cache, kbar,
                          lens, scale, out, idx, workspace, workspace_bytes, stream);
}

int bsattn_decode_ex(int dtype, int64_t B, int64_t Lmax, int Hq, int Hkv, int D, int block,
                     int topk, unsigned flags, const void* q, const void* k_cache,
                     const void* v_cache, const float* kbar, const int32_t* lens, float scale,
                     void* out, int32_t* idx, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int st = check_decode(dtype, B, Lmax, Hq, Hkv, D, block);
  if (st != BSATTN_OK) return st;
  if (flags & ~(unsigned)BSATTN_GROUP_SELECT)
    return fail(BSATTN_E_INVALID, "decode flags 0x%x (only BSATTN_GROUP_SELECT)", flags);
  if (topk < 1) return fail(BSATTN_E_INVALID, "topk %d must be >= 1", topk);
  if (!isfinite(scale) || !(scale > 0.f))
    return fail(BSATTN_E_INVALID, "scale must be finite and > 0");
  if (B == 0 || Lmax == 0) return BSATTN_OK;
  if (!q || !k_cache || !v_cache || !kbar || !lens || !out || !idx)
    return fail(BSATTN_E_INVALID, "null pointer argument");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(kbar) ||
      !aligned16(out) || ((uintptr_t)lens & 3u) || ((uintptr_t)idx & 3u))
    return fail(BSATTN_E_INVALID, "tensors must be 16-byte aligned, lens and idx 4-byte aligned");
  const size_t need = bsattn::decode_workspace_bytes(B, Hq, D, topk);
  if (!workspace || workspace_bytes < need)
    return fail(BSATTN_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if ((uintptr_t)workspace & 255u) return fail(BSATTN_E_WORKSPACE, "workspace not 256-byte aligned");
  return hip_status(bsattn::launch_decode(B, Lmax, Hq, Hkv, D, block, topk,
                                          flags & BSATTN_GROUP_SELECT, q, k_cache, v_cache,
                                          kbar, lens, scale, out, idx, workspace,
                                          (hipStream_t)stream),
                    "decode launch");
}

}  // extern "C"
