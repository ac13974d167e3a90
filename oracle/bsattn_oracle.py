"""fp64 CPU oracle for block-sparse attention with top-k block selection.

TEST INFRASTRUCTURE. Only the test suite, the smoke check of the package entry
and the bench's CPU-baseline leg may import this module. The HIP path never
imports it, and it imports nothing from the HIP path: the two share no code.
It is plain and slow on purpose: numpy in float64, a library matmul or sort as
a step, no blocking or fusion beyond what the definitions state.

Sources, cited by page title and section:
  [SF]  SparseFormer page, qqiyuan.cn, "2026 新一代卷积与Transformer网络架构技术演进与性能对比":
        section "SparseFormer 关键技术" (block-sparse attention: the N x N score matrix is
        cut into blocks and the important blocks are TopK(Q_B K_B^T / sqrt(d), k)), and
        section "SparseFormer 注意力实现" (block_sparse_attention(q, k, v, block_size,
        topk_ratio) on q/k/v [B, N, H, D] in three steps: 1 mean-pool q and k per block and
        form block scores with an einsum over d; 2 torch.topk with
        k = int(topk_ratio * num_blocks); 3 attention over the selected blocks only with
        scale 1/sqrt(D)).
  [MSA] MSA page, cloud.baidu.com, "从M2.7到M3：多模态模型稀疏注意力架构设计与实现全解析":
        §2.1 "核心数学模型" (sparse attention as Softmax(Mask(Q K^T / sqrt(d_k))) V, the mask
        deciding which positions take part), §2.2 (two stages: block-level scores, then full
        attention inside the chosen blocks), §3.1 (GQA-based attention block).

Readings where the pages are silent or garbled (each is listed with its reason in
the design notes of the repository):
  R1  pooled blocks are laid out [B, H, nb, D] before the score einsum, so scores are
      per (batch, head) [B, H, nb, nb] as the sketch's shape comments state;
  R2  block scores are the unscaled product of pooled blocks (the sketch's einsum); the
      1/sqrt(d) of the formula is a positive factor that leaves the order unchanged;
  R4  ties between equal scores go to the lower key-block index;
  R5  the selected indices of a row are returned in ascending block order;
  R7  N must be a multiple of the block size (the sketch's .view needs it);
  R8  no causal mask in the pages' method; the causal variant (R20) is an option;
  R10 GQA: query head h reads KV head h // (Hq // Hkv); selection is per query head;
  R15 fp8 inputs are OCP e4m3 ("fn": no infinities, S.1111.111 is NaN) codes times a
      per-tensor descale.
  R20 causal variant: query block i may select key blocks j <= i only; its own block i is
      always selected and the other min(k, i+1) - 1 places go to the best-scoring j < i
      (ties to the lower j); unused places of a row hold -1; inside the own block query t
      sees keys u <= t. (The MSA page names MoBA among the block-based methods and checks
      that weights concentrate near the diagonal; the pages give no causal rule.)
  R21 in-block max pooling: the "in-block extremum" scoring of the MSA page's §2.2 table
      read as the elementwise maximum over the block's tokens, for q and k alike.
  R22 group-shared selection (GQA, MSA §3.1): one selection per KV head from the sum of
      the block scores of its query heads (equivalently, from the summed pooled queries);
      every query head of the group uses it.
  R26 decode (the pages' KV cache and first-token latency remarks): one new query
      token per sequence against a cache of L tokens, the query at position L-1. Its own block
      (L-1) // b, complete or not, is always used; the other min(k, own+1) - 1 places go to
      the complete blocks j < own with the largest q . kbar_j (kbar: mean of the block's keys,
      kept up to date as blocks complete; ties to the lower j); attention over those blocks
      and the own block's cached tokens (all at positions <= L-1).
  R29 group-shared decode selection: with the option, one choice per (sequence, KV head) by
      the sum over its query heads of q_h . kbar_j (R22 for a single query token), used by
      each of those heads.
  R27 random blocks (the MSA page's §5.1 remedy "5% random blocks"): of a row's k
      places, k - r keep the best scores and r go to blocks drawn uniformly without
      replacement from the others: draw p (p < r) takes the (x mod m_p)-th remaining block in
      ascending order, m_p = nb - (k - r) - p, x = element row * 2^16 + p of the SplitMix64
      sequence (Steele, Lea, Flood, OOPSLA 2014) seeded with the caller's seed, row the
      row's position (batch, head, query block) in C order.
  R28 overlapping key blocks (the MSA page's §5.3 remedy for block-boundary effects,
      overlap ratio 0.25): key block j holds the b tokens from j*s on, cut at N, with the
      stride s = b - overlap*b (48 for b = 64, 96 for b = 128), and key blocks follow until one
      reaches the last token; query blocks stay the b-token partition. Pooling, scores and
      top-k run over the key blocks; a query block attends to the union of the tokens of its
      selected key blocks, each token once. The causal rule (R20) is not defined for them.
  R25 backward (the MSA page's §4.1 checks that back-propagation is complete; the
      SparseFormer page recommends the method for training large models, "千亿参数大模型训练"):
      gradients of the gathered-block attention with the selection held fixed (top-k is
      piecewise constant); the softmax Jacobian written out.

Every function below is pinned by the CPU tests (tests/test_oracle_*.py) against
closed forms, library routines, brute force or invariants; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Widening of stored values to float64
# ---------------------------------------------------------------------------


def widen_bf16_bits(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 value is the upper half of the float32 with the same bits.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):     # NaN payloads widen to NaN
        return b.view(np.float32).astype(np.float64)


def decode_e4m3(codes) -> np.ndarray:
    """OCP 8-bit floating point E4M3 codes (uint8) -> float64 [R15].

    Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits. Exponent field 0
    is subnormal: value = m/8 * 2^(1-7). Otherwise value = (1 + m/8) * 2^(e-7). The
    format has no infinities; exponent 15 with mantissa 7 is NaN, so the largest
    finite magnitude is (1 + 6/8) * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m / 8.0 * 2.0 ** (1 - 7)
    norm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    mag = np.where(e == 0, sub, norm)
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


def widen(x, dtype: str, descale: float = 1.0) -> np.ndarray:
    """Stored tensor (numpy array) -> float64 values the method sees.

    dtype "f32": float32 array; "bf16": uint16 bit patterns; "fp8": uint8 e4m3 codes,
    multiplied by the per-tensor descale (in float64).
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return widen_bf16_bits(x)
    if dtype == "fp8":
        return decode_e4m3(x) * np.float64(descale)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# The method, step by step
# ---------------------------------------------------------------------------


def topk_count(ratio: float, num_blocks: int) -> int:
    """k = int(topk_ratio * num_blocks) [SF "SparseFormer 注意力实现", step 2]."""
    return int(ratio * num_blocks)


def pool(x: np.ndarray, block: int) -> np.ndarray:
    """Mean of the `block` tokens of every block, per head [SF step 1; R1, R7].

    x: [B, N, H, D] float64 -> [B, H, nb, D] float64 with nb = N // block.
    """
    B, N, H, D = x.shape
    if N % block:
        raise ValueError("N must be a multiple of the block size")
    nb = N // block
    return x.reshape(B, nb, block, H, D).mean(axis=2).transpose(0, 2, 1, 3)


def pool_max(x: np.ndarray, block: int) -> np.ndarray:
    """Elementwise maximum over the `block` tokens of every block, per head [R21].

    x: [B, N, H, D] float64 -> [B, H, nb, D] float64.
    """
    B, N, H, D = x.shape
    if N % block:
        raise ValueError("N must be a multiple of the block size")
    nb = N // block
    return x.reshape(B, nb, block, H, D).max(axis=2).transpose(0, 2, 1, 3)


def key_block_ranges(N: int, block: int, stride: int):
    """Token ranges [start, end) of overlapping key blocks [R28].

    Key block j starts at token j * stride and holds `block` tokens, cut at N; blocks follow
    until one ends at N. stride == block gives the plain partition of `pool`. The stride
    lies in [block/2, block], so only neighbouring key blocks share tokens.
    """
    if not (0 < stride <= block and 2 * stride >= block):
        raise ValueError("the key stride must lie in [block/2, block]")
    ranges = []
    start = 0
    while N > 0:
        end = min(start + block, N)
        ranges.append((start, end))
        if end == N:
            break
        start += stride
    return ranges


def pool_key_blocks(x: np.ndarray, block: int, stride: int, pooling: str = "mean") -> np.ndarray:
    """Pooled overlapping key blocks [R28; R21 for "max"]: the mean (or elementwise maximum)
    of each key block's own tokens; a shorter last block is pooled over the tokens it has.

    x: [B, N, H, D] float64 -> [B, H, nw, D] float64, nw = len(key_block_ranges(...)).
    """
    reduce = np.mean if pooling == "mean" else np.max
    parts = [reduce(x[:, s:e], axis=1) for s, e in key_block_ranges(x.shape[1], block, stride)]
    return np.stack(parts, axis=2)


def union_tokens(sel, N: int, block: int, stride: int) -> np.ndarray:
    """Ascending token positions covered by the key blocks `sel` (entries -1 skipped), each
    position once [R28]."""
    ranges = key_block_ranges(N, block, stride)
    return np.unique(np.concatenate([np.arange(*ranges[j]) for j in sel if j >= 0]))


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h under GQA [MSA §3.1; R10]."""
    return h // (Hq // Hkv)


def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """S[b,h,i,j] = sum_d qbar[b,h,i,d] * kbar[b,kv(h),j,d], unscaled [SF step 1; R2].

    qbar [B, Hq, nb, D], kbar [B, Hkv, nb, D] -> S [B, Hq, nb, nb].
    """
    B, Hq, nb, D = qbar.shape
    Hkv = kbar.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    S = np.empty((B, Hq, nb, kbar.shape[2]), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            S[b, h] = qbar[b, h] @ kbar[b, kv_head(h, Hq, Hkv)].T
    return S


def select_topk(S: np.ndarray, k: int) -> np.ndarray:
    """Top-k key blocks of every score row [SF step 2; R4, R5].

    The k-th largest score T of a row is found with a partition; every entry above T
    is kept, and of the entries equal to T the ones with the lowest block index fill
    the remaining places. Returns int64 [..., k], ascending block index per row.
    """
    nb = S.shape[-1]
    if not 1 <= k <= nb:
        raise ValueError("k must lie in [1, nb]")
    T = -np.partition(-S, k - 1, axis=-1)[..., k - 1:k]     # k-th largest per row
    above = S > T
    equal = S == T
    need = k - above.sum(axis=-1, keepdims=True)
    rank_in_equal = np.cumsum(equal, axis=-1)                # 1-based, ascending j
    keep = above | (equal & (rank_in_equal <= need))
    rows = keep.reshape(-1, nb)
    idx = np.nonzero(rows)[1].reshape(S.shape[:-1] + (k,))
    return idx.astype(np.int64)


def select_topk_causal(S: np.ndarray, k: int) -> np.ndarray:
    """Causal selection [R20]: row i (the query block, second-to-last axis) keeps its own
    block i and the min(k, i+1) - 1 best blocks among j < i (ties to the lower j, as in
    `select_topk`); ascending order; places past min(k, i+1) hold -1.
    Returns int64 [..., nb, k].
    """
    nb = S.shape[-1]
    if S.shape[-2] != nb or not 1 <= k <= nb:
        raise ValueError("square score rows and k in [1, nb] required")
    out = np.full(S.shape[:-1] + (k,), -1, dtype=np.int64)
    for i in range(nb):
        ki = min(k, i + 1)
        row = out[..., i, :]
        if ki > 1:
            row[..., :ki - 1] = select_topk(S[..., i, :i], ki - 1)   # over j < i
        row[..., ki - 1] = i                                      # own block, largest index
    return out


_U64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed: int, n: int) -> int:
    """Element n (0-based) of the SplitMix64 sequence seeded with `seed`: the state after
    n + 1 Weyl steps of GAMMA, through the published 64-bit finaliser [R27]."""
    z = (seed + (n + 1) * _GAMMA) & _U64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _U64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _U64
    return z ^ (z >> 31)


def select_topk_random(S: np.ndarray, k: int, r: int, seed: int) -> np.ndarray:
    """Top k - r blocks by score plus r random others per row [R27]; ascending.

    S [..., nb]; the row number of S[..., :] is its position in C order over the leading axes.
    """
    nb = S.shape[-1]
    if not (1 <= k <= nb and 0 <= r <= k):
        raise ValueError("need 1 <= k <= nb and 0 <= r <= k")
    rows = S.reshape(-1, nb)
    out = np.empty((rows.shape[0], k), dtype=np.int64)
    for row in range(rows.shape[0]):
        top = select_topk(rows[row][None], k - r)[0].tolist() if k > r else []
        rest = [j for j in range(nb) if j not in set(top)]
        picked = []
        for p in range(r):
            x = splitmix64(seed, row * 65536 + p)
            picked.append(rest.pop(x % len(rest)))
        out[row] = sorted(top + picked)
    return out.reshape(S.shape[:-1] + (k,))


def group_scores(S: np.ndarray, Hkv: int) -> np.ndarray:
    """Block scores of a KV head group: the sum over its query heads [R22].

    S [B, Hq, nb, nb] -> [B, Hkv, nb, nb]; query heads g*G .. g*G+G-1 form group g.
    """
    B, Hq, nb, nbk = S.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return S.reshape(B, Hkv, Hq // Hkv, nb, nbk).sum(axis=2)


def kth_scores(S: np.ndarray, k: int):
    """(s_k, s_{k+1}): the k-th and (k+1)-th largest score of every row.

    s_{k+1} is -inf when k equals the row length.
    """
    srt = -np.sort(-S, axis=-1)
    sk = srt[..., k - 1]
    sk1 = srt[..., k] if k < S.shape[-1] else np.full(sk.shape, -np.inf)
    return sk, sk1


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray, block: int,
           scale: float, rows=None, causal: bool = False, stride=None) -> np.ndarray:
    """Exact softmax attention of every query block over its selected key blocks
    [SF step 3; MSA §2.1, §2.2; R8, R10; R20 when causal; R28 with a key stride].

    q [B, N, Hq, D], k/v [B, N, Hkv, D] float64; idx [B, Hq, nb, topk] (a set of key
    blocks per query block and head; entries -1 are unused places). For query t of block i
    the keys are the union of blocks idx[b,h,i,:] of KV head kv(h); weights
    softmax(scale * q_t . k_u); causal: only keys u <= t. stride: the key blocks overlap
    (`key_block_ranges`) and each token of the union counts once.
    rows: optional list of (b, h, i) to compute; the others are left NaN.
    Returns out [B, N, Hq, D] float64.
    """
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    nb = N // block
    if stride is not None and causal:
        raise ValueError("overlapping key blocks have no causal rule")
    out = np.full(q.shape, np.nan, dtype=np.float64)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(nb)]
    for (b, h, i) in rows:
        g = kv_head(h, Hq, Hkv)
        if stride is None:
            tok = np.concatenate([np.arange(j * block, (j + 1) * block)
                                  for j in idx[b, h, i] if j >= 0])
        else:
            tok = union_tokens(idx[b, h, i], N, block, stride)
        Qi = q[b, i * block:(i + 1) * block, h, :]           # [block, D]
        Ku = k[b, tok, g, :]                                 # [keys, D]
        Vu = v[b, tok, g, :]
        z = scale * (Qi @ Ku.T)
        if causal:
            t = np.arange(i * block, (i + 1) * block)
            z = np.where(tok[None, :] <= t[:, None], z, -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        out[b, i * block:(i + 1) * block, h, :] = (p @ Vu) / p.sum(axis=1, keepdims=True)
    return out


def attend_batched(q, k, v, idx, block, scale, bh=None, causal: bool = False) -> np.ndarray:
    """`attend` over all query blocks of the (b, h) pairs in `bh` at once.

    Same arithmetic as `attend` (gather the selected key blocks, scaled product,
    max-shifted exponent, weighted sum over the normaliser), with the gather and the
    products done for a whole (b, h) per library call. Unused places (-1) and, causal,
    keys after the query are masked with -inf. Used for large sizes only.
    """
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    nb = N // block
    out = np.full(q.shape, np.nan, dtype=np.float64)
    if bh is None:
        bh = [(b, h) for b in range(B) for h in range(Hq)]
    for (b, h) in bh:
        g = kv_head(h, Hq, Hkv)
        Kb = k[b, :, g, :].reshape(nb, block, D)
        Vb = v[b, :, g, :].reshape(nb, block, D)
        sel = idx[b, h]                                      # [nb, topk]
        used = sel >= 0
        safe = np.where(used, sel, 0)
        Ku = Kb[safe].reshape(nb, -1, D)                     # [nb, topk*block, D]
        Vu = Vb[safe].reshape(nb, -1, D)
        Qb = q[b, :, h, :].reshape(nb, block, D)
        z = scale * np.matmul(Qb, Ku.transpose(0, 2, 1))     # [nb, block, topk*block]
        keep = np.repeat(used, block, axis=1)[:, None, :]    # [nb, 1, topk*block]
        if causal:
            u = (safe[:, :, None] * block + np.arange(block)).reshape(nb, 1, -1)
            t = np.arange(N).reshape(nb, block, 1)
            keep = keep & (u <= t)
        z = np.where(keep, z, -np.inf)
        p = np.exp(z - z.max(axis=2, keepdims=True))
        o = np.matmul(p, Vu) / p.sum(axis=2, keepdims=True)
        out[b, :, h, :] = o.reshape(N, D)
    return out


def dense_attention(q, k, v, scale, causal: bool = False) -> np.ndarray:
    """Full softmax(scale * Q K^T) V per head [MSA §2.1, full-attention mask]; causal:
    query t sees keys u <= t only."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    out = np.empty(q.shape, dtype=np.float64)
    lower = np.tril(np.ones((N, N), dtype=bool))
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            z = scale * (q[b, :, h, :] @ k[b, :, g, :].T)
            if causal:
                z = np.where(lower, z, -np.inf)
            p = np.exp(z - z.max(axis=1, keepdims=True))
            out[b, :, h, :] = (p @ v[b, :, g, :]) / p.sum(axis=1, keepdims=True)
    return out


def masked_attention_bruteforce(q, k, v, idx, block, scale, causal: bool = False,
                                stride=None) -> np.ndarray:
    """Softmax(Mask(scale * Q K^T)) V with an explicit N x N token mask [MSA §2.1].

    M[t, u] is true when key u's block is among the blocks selected for query t's
    block (and, causal, u <= t); with a key stride [R28], when u lies in the token range of
    a selected key block. Masked positions get -inf before the softmax. Tiny sizes only.
    """
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    out = np.empty(q.shape, dtype=np.float64)
    tb = np.arange(N) // block
    ranges = key_block_ranges(N, block, stride) if stride is not None else None
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            M = np.zeros((N, N), dtype=bool)
            for t in range(N):
                if ranges is None:
                    M[t] = np.isin(tb, idx[b, h, tb[t]])
                else:
                    for j in idx[b, h, tb[t]]:
                        if j >= 0:
                            M[t, ranges[j][0]:ranges[j][1]] = True
                if causal:
                    M[t, t + 1:] = False
            z = np.where(M, scale * (q[b, :, h, :] @ k[b, :, g, :].T), -np.inf)
            p = np.exp(z - z.max(axis=1, keepdims=True))
            out[b, :, h, :] = (p @ v[b, :, g, :]) / p.sum(axis=1, keepdims=True)
    return out


def attend_lse(q, k, idx, block, scale, causal: bool = False) -> np.ndarray:
    """Natural log-sum-exp of every query row's scaled scores over its selected keys
    [SF step 3; R20 when causal]: lse[b, h, t] = log sum_u exp(scale * q_t . k_u).
    Returns [B, Hq, N] float64.
    """
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    nb = N // block
    lse = np.empty((B, Hq, N), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            for i in range(nb):
                tok = np.concatenate([np.arange(j * block, (j + 1) * block)
                                      for j in idx[b, h, i] if j >= 0])
                z = scale * (q[b, i * block:(i + 1) * block, h, :] @ k[b, tok, g, :].T)
                if causal:
                    t = np.arange(i * block, (i + 1) * block)
                    z = np.where(tok[None, :] <= t[:, None], z, -np.inf)
                m = z.max(axis=1)
                lse[b, h, i * block:(i + 1) * block] = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return lse


def attend_backward(q, k, v, idx, block, scale, dout, causal: bool = False):
    """Gradients of the gathered-block attention with the selection held fixed:
    for query block i with selected keys U, P = softmax(scale * Q_i K_U^T) (masked when
    causal), O_i = P V_U, and for the upstream gradient dO_i:
        dV_U += P^T dO_i,   dP = dO_i V_U^T,   dS = P * (dP - rowsum(dO_i * O_i)),
        dQ_i = scale * dS K_U,   dK_U += scale * dS^T Q_i
    (the softmax Jacobian written out). GQA: K/V gradients of KV head g collect the
    contributions of all its query heads. Returns (dq, dk, dv) float64 with the shapes of
    q, k, v.
    """
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    nb = N // block
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            for i in range(nb):
                rows = slice(i * block, (i + 1) * block)
                tok = np.concatenate([np.arange(j * block, (j + 1) * block)
                                      for j in idx[b, h, i] if j >= 0])
                Qi, dOi = q[b, rows, h, :], dout[b, rows, h, :]
                Ku, Vu = k[b, tok, g, :], v[b, tok, g, :]
                z = scale * (Qi @ Ku.T)
                if causal:
                    t = np.arange(i * block, (i + 1) * block)
                    z = np.where(tok[None, :] <= t[:, None], z, -np.inf)
                p = np.exp(z - z.max(axis=1, keepdims=True))
                P = p / p.sum(axis=1, keepdims=True)
                Oi = P @ Vu
                dP = dOi @ Vu.T
                dS = P * (dP - (dOi * Oi).sum(axis=1, keepdims=True))
                dq[b, rows, h, :] = scale * (dS @ Ku)
                np.add.at(dk[b, :, g, :], tok, scale * (dS.T @ Qi))
                np.add.at(dv[b, :, g, :], tok, P.T @ dOi)
    return dq, dk, dv


def decode_select(q_tok, kbar, lens, block: int, topk: int, group: bool = False) -> np.ndarray:
    """Blocks for one decode step [R26]. q_tok [B, Hq, D]; kbar [B, Hkv, nb, D] (rows of
    complete blocks are read); lens [B] (1 <= lens[b]). Returns int64 [B, Hq, topk]:
    ascending, own block last, -1 in unused places. group: one choice per KV head from the
    sum of its query heads' scores, used by each of them [R29].
    """
    B, Hq, D = q_tok.shape
    Hkv = kbar.shape[1]
    out = np.full((B, Hq, topk), -1, dtype=np.int64)
    for b in range(B):
        own = (int(lens[b]) - 1) // block
        kb = min(topk, own + 1)
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            if kb > 1:
                if group:
                    heads = [x for x in range(Hq) if kv_head(x, Hq, Hkv) == g]
                    s = sum(kbar[b, g, :own] @ q_tok[b, x] for x in heads)        # [own]
                else:
                    s = kbar[b, g, :own] @ q_tok[b, h]                            # [own]
                out[b, h, :kb - 1] = select_topk(s[None], kb - 1)[0]
            out[b, h, kb - 1] = own
    return out


def decode_attend(q_tok, k_cache, v_cache, idx, lens, block: int, scale: float) -> np.ndarray:
    """Attention of each sequence's newest token over its decode blocks [R26]: keys of the
    selected blocks (-1 unused), the own block only up to position lens[b] - 1.
    q_tok [B, Hq, D], caches [B, Lmax, Hkv, D] -> out [B, Hq, D]."""
    B, Hq, D = q_tok.shape
    Hkv = k_cache.shape[2]
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            tok = np.concatenate([np.arange(j * block, min((j + 1) * block, L))
                                  for j in idx[b, h] if j >= 0])
            z = scale * (k_cache[b, tok, g] @ q_tok[b, h])
            p = np.exp(z - z.max())
            out[b, h] = (p @ v_cache[b, tok, g]) / p.sum()
    return out


def select(q, k, block: int, topk: int, causal: bool = False, pooling: str = "mean",
           group: bool = False, nrand: int = 0, seed: int = 0, stride=None) -> np.ndarray:
    """Steps 1-2 [SF]: pool q and k, score the blocks, keep the top-k per row.

    causal [R20], pooling "mean" [SF] or "max" [R21], group: one selection per KV head
    group, repeated for each of its query heads [R22], nrand random places [R27] (not with
    causal), stride: overlapping key blocks [R28] (not with causal). Returns
    [B, Hq, nb, topk] (entries index key blocks).
    """
    pf = pool if pooling == "mean" else pool_max
    if stride is None:
        kbar = pf(k, block)
    else:
        if causal:
            raise ValueError("overlapping key blocks have no causal rule")
        kbar = pool_key_blocks(k, block, stride, pooling)
    S = block_scores(pf(q, block), kbar)
    Hq, Hkv = q.shape[2], k.shape[2]
    if group:
        S = group_scores(S, Hkv)
    if nrand:
        if causal:
            raise ValueError("random places are defined for the non-causal selection")
        idx = select_topk_random(S, topk, nrand, seed)
    else:
        idx = select_topk_causal(S, topk) if causal else select_topk(S, topk)
    if group:
        idx = np.repeat(idx, Hq // Hkv, axis=1)
    return idx


def block_sparse_attention(q, k, v, block_size=64, topk_ratio=0.3, scale=None):
    """The whole method [SF "SparseFormer 注意力实现"]: returns (out, idx).

    q [B, N, Hq, D], k/v [B, N, Hkv, D] float64; scale defaults to 1/sqrt(D).
    """
    B, N, Hq, D = q.shape
    nb = N // block_size
    topk = topk_count(topk_ratio, nb)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    idx = select(q, k, block_size, topk)
    return attend(q, k, v, idx, block_size, scale), idx
