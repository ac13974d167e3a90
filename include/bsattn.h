/*
 * bsattn.h -- C ABI of the MI355X (gfx950) block-sparse top-k attention library.
 *
 * The method (block-sparse attention with top-k block selection):
 *   SparseFormer page, qqiyuan.cn, "2026 新一代卷积与Transformer网络架构技术演进与性能对比",
 *   sections "SparseFormer 关键技术" (TopK over block scores) and "SparseFormer 注意力实现"
 *   (three steps: mean-pool q/k per block and score blocks; keep the top
 *   k = int(topk_ratio * num_blocks) key blocks per query block and head; attention over
 *   the selected blocks only with scale 1/sqrt(D)).
 *   MSA page, cloud.baidu.com, "从M2.7到M3：多模态模型稀疏注意力架构设计与实现全解析",
 *   §2.1 (Softmax(Mask(Q K^T / sqrt(d_k))) V), §2.2 (select blocks, then full attention
 *   inside them), §3.1 (GQA-based attention block).
 *
 * Conventions shared by every entry point
 *   - Tensors are contiguous, row-major, in device memory (HBM) owned by the caller.
 *     q is [B, N, Hq, D]; k and v are [B, N, Hkv, D]; out is [B, N, Hq, D];
 *     idx is [B, Hq, nb, topk] int32 with nb = N / block.
 *   - GQA: query head h reads KV head h / (Hq / Hkv); selection is per query head.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null stream),
 *     never synchronises (except the optional idx validation of bsattn_forward), never
 *     allocates or frees device memory, and keeps no state between calls (the static
 *     scratch of bsattn_select_noalloc aside). Argument checks
 *     run on the host before any launch.
 *   - Errors are returned, never thrown or printed: the return value is a bsattn_status;
 *     bsattn_last_error() gives a text detail of the last failure on the calling thread.
 *     Launch failures come back as BSATTN_E_HIP. Kernel faults surface at the caller's
 *     next synchronisation.
 *   - Supported now: D in {64, 128}; block in {64, 128}; storage dtypes fp32, bf16 and OCP
 *     fp8 e4m3 (fp8 attention: D = 128). Selection: nb <= 1024, or nb a multiple of 64 up
 *     to 8192 (the score matrix then goes through the workspace; group selection needs
 *     nb <= 1024). Other sizes give BSATTN_E_UNSUPPORTED.
 *   - B == 0 or N == 0 is an empty call: arguments are checked, nothing is launched
 *     (topk must then be 0 when nb == 0).
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSATTN_ABI_VERSION 5

typedef enum {
  BSATTN_OK = 0,
  BSATTN_E_INVALID = 1,      /* bad shape, pointer, alignment, topk or scale */
  BSATTN_E_UNSUPPORTED = 2,  /* valid arguments without a kernel (D, block, nb, dtype) */
  BSATTN_E_WORKSPACE = 3,    /* workspace missing or smaller than bsattn_select_workspace_bytes */
  BSATTN_E_HIP = 4           /* a HIP runtime call or kernel launch failed */
} bsattn_status;

typedef enum {
  BSATTN_F32 = 0,       /* IEEE binary32 */
  BSATTN_BF16 = 1,      /* bfloat16 */
  BSATTN_FP8_E4M3 = 2   /* OCP 8-bit E4M3 ("fn": no infinities), values = code * descale */
} bsattn_dtype;

/* Options of the extended entry points (bit flags, combine with |). */
/* Causal variant: query block i may select only key blocks j <= i; its own block i is always
 * selected, the other min(topk, i+1) - 1 places go to the best-scoring j < i (ties to the
 * lower j), the row stays ascending and its unused places hold -1; attention reads the
 * first min(topk, i+1) entries of the row, which must lie in [0, i], and inside block i
 * query t sees keys u <= t only. (The pages give no causal rule; the MSA page names MoBA
 * among the block-based methods and checks that weights concentrate near the diagonal.) */
#define BSATTN_CAUSAL 1u
/* Selection only: pool with the elementwise maximum over the block's tokens instead of the
 * mean (the "in-block extremum" scoring of the MSA page's §2.2 table). */
#define BSATTN_POOL_MAX 2u
/* Selection only (GQA, MSA page §3.1): one selection per KV head, from the sum over its
 * Hq/Hkv query heads of their block scores; it is written to the idx rows of each of those
 * heads. The workspace's pooled-query rows of the group's first head then hold the summed
 * pooled queries. For nb > 1024 the score matrix part of the workspace holds one
 * [nb, nb] matrix per (batch, KV head). */
#define BSATTN_GROUP_SELECT 4u

/* Version of this ABI (BSATTN_ABI_VERSION of the built library). Version 2 added the
 * BSATTN_* option flags, the two _ex entry points (with the optional log-sum-exp output) and
 * the backward; version 3 added the key_stride argument of the _ex entry points (overlapping
 * key blocks), bsattn_key_blocks and bsattn_select_workspace_bytes_ex; version 4 added
 * bsattn_decode_ex (group-shared decode selection); version 5 added bsattn_select_noalloc and
 * moved the measurement probes to their own library (include/bsattn_probe.h). Version-1
 * calls are unchanged. */
int bsattn_abi_version(void);

/* Static English text of a status code; never NULL. */
const char* bsattn_status_str(int status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). The
 * string is owned by the library and valid until the next call on that thread. */
const char* bsattn_last_error(void);

/* Bytes of device workspace bsattn_select needs for these sizes (0 for an empty call).
 * Layout, each part 256-byte aligned: pooled q, fp32 [B, Hq, nb, D]; then pooled k,
 * fp32 [B, Hkv, nb, D]; when nb > 1024 also the score matrix, fp32 [B, Hq, nb, nb]
 * (MSA page §3.2: 1M tokens at block 128 give 8192 key blocks per row), of which the causal
 * selection writes only the 128 x 128 tiles on and below the diagonal (its rows read no
 * other score). For fp8 inputs the pooled values are means of the e4m3 codes'
 * values without the per-tensor descale (a positive factor that does not change the
 * selection). Returns 0 and records an error for invalid sizes. */
size_t bsattn_select_workspace_bytes(int64_t B, int64_t N, int Hq, int Hkv, int D, int block);

/* Overlapping key blocks (the MSA page's §5.3 remedy for block-boundary effects: overlapping
 * blocks with overlap ratio 0.25). With key_stride s (block/2 <= s <= block; 0 means block),
 * key block j holds the tokens [j*s, min(j*s + block, N)): key blocks follow until one ends at
 * token N, so there are ceil((N - block) / s) + 1 of them (N / block when s == block). Query
 * blocks stay the N / block blocks of `block` tokens. The selection pools, scores and picks
 * key blocks (a shorter last block is pooled over its own tokens); attention of a query block
 * runs over the union of the tokens of its key blocks, each token once. Returns the number of
 * key blocks, or -1 (error recorded) for N < 0, N % block != 0 or a stride outside
 * [block/2, block]. */
int64_t bsattn_key_blocks(int64_t N, int block, int key_stride);

/* bsattn_select_workspace_bytes for key blocks at key_stride (0: block): the pooled-k part is
 * fp32 [B, Hkv, bsattn_key_blocks(N, block, key_stride), D]. */
size_t bsattn_select_workspace_bytes_ex(int64_t B, int64_t N, int Hq, int Hkv, int D, int block,
                                        int key_stride);

/*
 * Block selection (steps 1-2 of "SparseFormer 注意力实现" on the SparseFormer page).
 *   Pooled blocks: qbar[b,h,i,:] = mean of q[b, i*block + t, h, :] over t < block, and kbar
 *   likewise per KV head, accumulated in fp32.
 *   Scores: S[b,h,i,j] = sum_d qbar[b,h,i,d] * kbar[b,h/(Hq/Hkv),j,d], fp32, unscaled (the
 *   1/sqrt(d) of the page's formula is a positive factor and leaves the order unchanged).
 *   idx[b,h,i,:] = the topk key blocks j with the largest S[b,h,i,j]; equal scores go to the
 *   lower j (-0.0 equals +0.0); written in ascending j. NaN scores are unspecified.
 * Arguments
 *   dtype      bsattn_dtype of q and k.
 *   B, N       batch and sequence length; N % block == 0.
 *   Hq, Hkv    query and KV heads; Hq % Hkv == 0.
 *   D          head dimension.
 *   block      tokens per block.
 *   topk       1 <= topk <= nb (callers of the page's form pass int(topk_ratio * nb)).
 *   q, k       device pointers, 16-byte aligned.
 *   idx        device pointer, int32 [B, Hq, nb, topk], written entirely.
 *   workspace  device pointer, 256-byte aligned, at least bsattn_select_workspace_bytes.
 *   stream     hipStream_t.
 */
int bsattn_select(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                  const void* q, const void* k, int32_t* idx,
                  void* workspace, size_t workspace_bytes, void* stream);

/* bsattn_select with options: flags is a combination of BSATTN_CAUSAL, BSATTN_POOL_MAX and
 * BSATTN_GROUP_SELECT (0 gives bsattn_select). Other bits: BSATTN_E_INVALID. Workspace:
 * bsattn_select_workspace_bytes_ex with the same key_stride.
 *   nrand  random places (the MSA page's §5.1 remedy "5% random blocks"; 0: none): each row
 *          keeps its topk - nrand best blocks, then draw p = 0 .. nrand-1 takes the
 *          (x mod m_p)-th of the m_p = nb - (topk - nrand) - p blocks not yet chosen, in
 *          ascending order, with x = element row * 65536 + p of the SplitMix64 sequence
 *          (Steele, Lea, Flood, OOPSLA 2014) seeded with `seed`; row = (b * S + s) * nb + i
 *          for selection head s of S (S = Hq, or Hkv with BSATTN_GROUP_SELECT). The row stays
 *          ascending. 0 <= nrand <= topk (else BSATTN_E_INVALID); not with BSATTN_CAUSAL and
 *          only for nb <= 1024 (else BSATTN_E_UNSUPPORTED). With overlapping key blocks the
 *          draws run over the key blocks (nb above reads bsattn_key_blocks).
 *   seed   the generator's seed.
 *   key_stride  0 or block: the plain blocks. Otherwise overlapping key blocks (see
 *          bsattn_key_blocks; stride outside [block/2, block]: BSATTN_E_INVALID): idx rows name
 *          key blocks, 1 <= topk <= bsattn_key_blocks(...); not with BSATTN_CAUSAL and for at
 *          most 1024 key blocks (else BSATTN_E_UNSUPPORTED).
 * Arguments, layouts and errors otherwise as bsattn_select. */
int bsattn_select_ex(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block,
                     int topk, unsigned flags, int nrand, uint64_t seed, int key_stride,
                     const void* q, const void* k, int32_t* idx, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * bsattn_select_ex without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The pooled blocks (and, for nb > 1024, the score matrix) go to a static
 * device array of bsattn_select_noalloc_max_bytes() bytes (64 MiB) that the library holds on
 * every GPU it runs on until the process ends; its address is looked up once per device.
 * The call allocates nothing. Arguments, layouts and errors as bsattn_select_ex; a selection
 * whose workspace (bsattn_select_workspace_bytes_ex) exceeds the static size returns
 * BSATTN_E_WORKSPACE before any HIP call. Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (other streams, other threads) race; calls in one
 * stream are ordered. Nothing in the array needs to start at zero.
 */
size_t bsattn_select_noalloc_max_bytes(void);
int bsattn_select_noalloc(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block,
                          int topk, unsigned flags, int nrand, uint64_t seed, int key_stride,
                          const void* q, const void* k, int32_t* idx, void* stream);

/*
 * Gathered-block attention (step 3 of "SparseFormer 注意力实现"; MSA page §2.1 with a
 * block mask, §2.2 second stage).
 *   For query token t of block i and query head h, with g = h / (Hq / Hkv):
 *   out[b,t,h,:] = sum over keys u in the blocks idx[b,h,i,:] of
 *                  softmax_u(scale * q[b,t,h,:] . k[b,u,g,:]) * v[b,u,g,:].
 *   Scores and the softmax state are fp32; fp32 inputs compute in fp32, bf16 inputs multiply
 *   on bf16 MFMA with the probabilities rounded to bf16, fp8 inputs multiply on the fp8 MFMA
 *   with the probabilities rounded to e4m3 (values = codes * descale_qkv).
 * Arguments
 *   dtype, B, N, Hq, Hkv, D, block, topk  as for bsattn_select.
 *   q, k, v      device pointers, 16-byte aligned.
 *   idx          device pointer, int32 [B, Hq, nb, topk]; each row should hold distinct
 *                blocks in [0, nb). A row with an out-of-range entry is not read out of
 *                bounds: its output rows are set to NaN. Duplicate entries count twice.
 *                With BSATTN_VALIDATE=1 in the environment every row is first checked on
 *                the GPU (strictly ascending, in [0, nb)); a failing row makes the call
 *                return BSATTN_E_INVALID before the attention launch (the first 4 bytes of
 *                out then hold the check's row count, the rest of out is untouched). This
 *                mode waits for the stream.
 *   scale        finite softmax scale (the page uses 1/sqrt(D)).
 *   descale_qkv  host pointer to 3 floats (q, k, v per-tensor descales) for fp8; ignored
 *                (may be NULL) for other dtypes. Must be finite and > 0.
 *   out          device pointer, 16-byte aligned: fp32 for fp32 inputs, bf16 for bf16 and
 *                fp8 inputs; [B, N, Hq, D], written entirely.
 *   stream       hipStream_t.
 */
int bsattn_forward(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                   const void* q, const void* k, const void* v, const int32_t* idx,
                   float scale, const float* descale_qkv, void* out, void* stream);

/* bsattn_forward with options: BSATTN_CAUSAL gives the causal variant (row i reads its first
 * min(topk, i+1) entries, each in [0, i]; an entry outside makes that query block's output
 * NaN; keys after the query inside block i are masked). The selection-only bits
 * BSATTN_POOL_MAX and BSATTN_GROUP_SELECT are accepted and have no effect here; other bits:
 * BSATTN_E_INVALID. Under BSATTN_VALIDATE=1 causal rows are checked in that form (unused
 * places must hold -1).
 *   key_stride  0 or block: the plain blocks. Otherwise idx rows name overlapping key blocks
 *        (bsattn_key_blocks) in [0, key blocks) and each query block attends to the union of
 *        their tokens, every token once (rows should name distinct blocks); not with
 *        BSATTN_CAUSAL and for at most 8192 key blocks (else BSATTN_E_UNSUPPORTED).
 *   lse  optional device pointer (NULL: not written), fp32 [B, Hq, N], 4-byte aligned: the
 *        natural log-sum-exp of every query row's scaled scores over its keys,
 *        log sum_u exp(scale * q_t . k_u) (for fp8, of the descaled values); NaN for a row
 *        whose idx entry was out of range. bsattn_backward takes it.
 * Arguments, layouts and errors otherwise as bsattn_forward. */
int bsattn_forward_ex(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block,
                      int topk, unsigned flags, int key_stride, const void* q, const void* k,
                      const void* v, const int32_t* idx, float scale, const float* descale_qkv,
                      void* out, float* lse, void* stream);

/* Bytes of device workspace bsattn_backward needs (0 for an empty call): Dvec fp32
 * [B, Hq, N], key-block offsets int32 [B, Hkv, nb + 1], pair lists int32 [B, Hq, nb, topk],
 * each part 256-byte aligned; for block 128 those of the 64-token form (nb = N / 64, 2 * topk
 * places) followed by its index rows, int32 [B, Hq, N / 64, 2 * topk]. Returns 0 and records
 * an error for invalid sizes. */
size_t bsattn_backward_workspace_bytes(int64_t B, int64_t N, int Hq, int Hkv, int D, int block,
                                       int topk);

/*
 * Backward of bsattn_forward(_ex) with the selection held fixed (the top-k choice is piecewise
 * constant in q and k). SparseFormer page: the method is recommended for training large
 * models; MSA page §4.1 checks that back-propagation through the sparse attention is complete.
 * For query block i with keys U (its selected blocks; causal: masked as in the forward),
 * P = softmax(scale * Q_i K_U^T), O_i = P V_U and the upstream gradient dO_i:
 *   dV_U += P^T dO_i, dP = dO_i V_U^T, dS = P * (dP - rowsum(dO_i * O_i)),
 *   dQ_i = scale * dS K_U, dK_U += scale * dS^T Q_i
 * (GQA: a KV head collects the contributions of all its query heads).
 * Supported: dtype BSATTN_BF16, D in {64, 128}, block 64 or 128, N / 64 <= 4096, the plain
 * key blocks (a forward with key_stride 0 or block); other combinations give
 * BSATTN_E_UNSUPPORTED. Block 128 runs as 64-token blocks: each 128-token query block as two
 * 64-row halves over both halves of every selected block (the same key set per query), the
 * index rows of that form written to the workspace first. Products on bf16 MFMA with fp32 accumulation (P and dS rounded to bf16
 * as MFMA operands); the key-side sums run in a fixed order, so results are reproducible.
 * Arguments
 *   dtype .. topk, flags  as for bsattn_forward_ex (BSATTN_CAUSAL selects the causal variant;
 *                the other bits have no effect).
 *   q, k, v, idx, out    the forward's inputs and output (out: bf16 [B, N, Hq, D]); idx rows
 *                must name distinct blocks (as bsattn_select writes them); an out-of-range
 *                entry is skipped (never read out of bounds).
 *   dout         device pointer, bf16 [B, N, Hq, D]: gradient of the loss w.r.t. out.
 *   lse          device pointer, fp32 [B, Hq, N]: as written by bsattn_forward_ex.
 *   scale        the forward's scale (finite, > 0).
 *   dq           device pointer, fp32 [B, N, Hq, D], written entirely.
 *   dk, dv       device pointers, fp32 [B, N, Hkv, D], written entirely (0 for keys no query
 *                block selected).
 *   workspace    device pointer, 256-byte aligned, at least bsattn_backward_workspace_bytes.
 *   stream       hipStream_t.
 * Tensors 16-byte aligned; idx and lse 4-byte aligned.
 */
int bsattn_backward(int dtype, int64_t B, int64_t N, int Hq, int Hkv, int D, int block, int topk,
                    unsigned flags, const void* q, const void* k, const void* v,
                    const int32_t* idx, const void* out, const void* dout, const float* lse,
                    float scale, float* dq, float* dk, float* dv, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * Decode (one new query token per sequence against a KV cache).
 * Caches: k_cache, v_cache bf16 [B, Lmax, Hkv, D] (token t of sequence b at row t), pooled
 * keys kbar fp32 [B, Hkv, D, Lmax / block] (transposed: kbar[b,g,:,j] = mean of the keys of
 * block j once that block is complete), lens int32 [B] on the device: tokens cached per sequence
 * (1 <= lens[b] <= Lmax; the query is token lens[b] - 1, its K and V already in the cache).
 * SparseFormer page, "SparseFormer 注意力实现" (pooled key blocks, top-k blocks, attention over
 * them with scale 1/sqrt(D)); MSA page §5.2 (first-token latency of the block scoring).
 * Supported: dtype BSATTN_BF16, D in {64, 128}, block in {64, 128}, Lmax / block <= 8192,
 * B <= 65535; else BSATTN_E_UNSUPPORTED. Asynchronous on `stream`, no allocation.
 */

/* Pools the blocks completed between two lengths: for every sequence b, the blocks
 * j with lens_old[b] / block <= j < lens_new[b] / block get kbar rows (fp32 means of their
 * keys, all KV heads). lens_old may be NULL (then every complete block is pooled). Sequences
 * with an invalid length pair are skipped. k_cache, kbar 16-byte aligned. */
int bsattn_decode_pool(int dtype, int64_t B, int64_t Lmax, int Hkv, int D, int block,
                       const void* k_cache, const int32_t* lens_old, const int32_t* lens_new,
                       float* kbar, void* stream);

/* Bytes of device workspace bsattn_decode needs (per-split partial results, fp32). */
size_t bsattn_decode_workspace_bytes(int64_t B, int Hq, int D, int topk);

/* One decode step for every sequence and query head h (KV head h / (Hq / Hkv)):
 *   own = (lens[b] - 1) / block is always used; the other min(topk, own + 1) - 1 places go to
 *   the complete blocks j < own with the largest sum_d q[b,h,d] * kbar[b,g,d,j] (fp32;
 *   ties to the lower j); idx[b,h,:] receives them ascending (own last), then -1.
 *   out[b,h,:] = softmax over the keys of those blocks (own block: positions < lens[b]) of
 *   scale * q . k, times v; bf16 [B, Hq, D]; fp32 scores and sums.
 * q bf16 [B, Hq, D]; idx int32 [B, Hq, topk] written; workspace at least
 * bsattn_decode_workspace_bytes, 256-byte aligned. A sequence with lens[b] outside
 * [1, Lmax] gets idx -1 and NaN output. */
int bsattn_decode(int dtype, int64_t B, int64_t Lmax, int Hq, int Hkv, int D, int block, int topk,
                  const void* q, const void* k_cache, const void* v_cache, const float* kbar,
                  const int32_t* lens, float scale, void* out, int32_t* idx, void* workspace,
                  size_t workspace_bytes, void* stream);

/* bsattn_decode with options: flags 0 gives bsattn_decode; BSATTN_GROUP_SELECT makes one
 * choice per (sequence, KV head) from the sum over its Hq/Hkv query heads of their scores
 * (sum_d (sum_h q[b,h,d]) * kbar[b,g,d,j]; the MSA page's §3.1 GQA, as for bsattn_select_ex),
 * written to the idx rows of each of those heads, which then read the same blocks (the
 * attention runs them side by side, so their keys and values are fetched once). Other bits:
 * BSATTN_E_INVALID. Arguments, layouts and errors otherwise as bsattn_decode. */
int bsattn_decode_ex(int dtype, int64_t B, int64_t Lmax, int Hq, int Hkv, int D, int block,
                     int topk, unsigned flags, const void* q, const void* k_cache,
                     const void* v_cache, const float* kbar, const int32_t* lens, float scale,
                     void* out, int32_t* idx, void* workspace, size_t workspace_bytes,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
