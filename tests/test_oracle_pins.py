"""Pins of the fp64 oracle against things other than itself.

Each pin checks one oracle function against a closed form, a library routine
computed independently (torch in float64 on the CPU), brute force on tiny
inputs, or an invariant the mathematics fixes. The planted-mistake tests at the
end make sure a plausible error in the oracle (dropped term, wrong index, wrong
sign, transposed operand, wrong tie rule) fails at least one pin.
"""
import fractions
import math
import os

import numpy as np
import pytest
import torch

import oracle.bsattn_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def rng(seed):
    return np.random.default_rng(seed)


def rand_qkv(B, N, Hq, Hkv, D, seed=0):
    r = rng(seed)
    return (r.standard_normal((B, N, Hq, D)), r.standard_normal((B, N, Hkv, D)),
            r.standard_normal((B, N, Hkv, D)))


# ---------------------------------------------------------------- pin checks
# Each check raises AssertionError when the oracle disagrees with the pin.

def check_bf16_widen(o=O):
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits.astype(np.uint32) >> 7) & 0xFF) != 0xFF
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = o.widen_bf16_bits(bits)
    assert np.array_equal(got[finite], ref[finite])
    # closed forms
    assert o.widen_bf16_bits([0x3F80])[0] == 1.0
    assert o.widen_bf16_bits([0xC000])[0] == -2.0
    assert o.widen_bf16_bits([0x0001])[0] == 2.0 ** -133
    assert o.widen_bf16_bits([0x7F7F])[0] == (2 - 2.0 ** -7) * 2.0 ** 127


def check_e4m3(o=O):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = o.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # closed forms from the format's definition
    assert o.decode_e4m3([0x7E])[0] == 448.0
    assert o.decode_e4m3([0x38])[0] == 1.0
    assert o.decode_e4m3([0x01])[0] == 2.0 ** -9
    assert o.decode_e4m3([0x08])[0] == 2.0 ** -6
    assert o.decode_e4m3([0xBC])[0] == -1.5
    assert np.isnan(o.decode_e4m3([0x7F])[0]) and np.isnan(o.decode_e4m3([0xFF])[0])
    assert int(nan.sum()) == 2


def check_widen(o=O):
    """widen() per dtype: fp32 and bf16 exactly; fp8 codes times a non-unit descale, against
    torch's e4m3 decoding (a library routine) and a quantise/widen round trip that must land
    within e4m3 rounding of the value it started from [R15]."""
    x32 = rng(11).standard_normal(64).astype(np.float32)
    assert np.array_equal(o.widen(x32, "f32"), x32.astype(np.float64))
    bits = rng(12).integers(0, 1 << 15, 64).astype(np.uint16)
    assert np.array_equal(o.widen(bits, "bf16"),
                          torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
                          .to(torch.float64).numpy())
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for d in (0.37, 1.0 / 448.0, 3.0):
        assert np.array_equal(o.widen(codes, "fp8", d), lib * d)
    # round trip: per-tensor amax scaling to 448, e4m3 rounding (torch, nearest even), widen
    x = torch.from_numpy(rng(13).standard_normal(4096) * 2.5)
    amax = float(x.abs().max())
    q8 = (x * (448.0 / amax)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    back = o.widen(q8, "fp8", amax / 448.0)
    xs = x.numpy()
    # normal e4m3 values (|x| >= 2^-6 before descaling) carry relative error <= 2^-4; the
    # subnormal spacing is 2^-9, so the absolute error there is <= 2^-10 (times the descale)
    tol = np.maximum(2.0 ** -4 * np.abs(xs), 2.0 ** -10 * amax / 448.0) * (1 + 1e-12)
    assert np.all(np.abs(back - xs) <= tol)
    assert np.sqrt(np.mean((back - xs) ** 2)) < 0.05 * np.sqrt(np.mean(xs ** 2))


def check_pool(o=O):
    B, N, H, D, blk = 2, 24, 3, 5, 4
    x = rng(1).standard_normal((B, N, H, D))
    got = o.pool(x, blk)
    assert got.shape == (B, H, N // blk, D)
    for b in range(B):               # brute force, pure Python sums
        for h in range(H):
            for i in range(N // blk):
                for d in range(D):
                    s = 0.0
                    for t in range(blk):
                        s += x[b, i * blk + t, h, d]
                    assert abs(got[b, h, i, d] - s / blk) <= 1e-15 * blk
    c = np.full((1, 8, 2, 3), 0.375)
    assert np.all(o.pool(c, 4) == 0.375)      # a constant block pools to itself


def check_scores(o=O):
    B, Hq, Hkv, nb, D = 2, 4, 2, 5, 3
    r = rng(2)
    qb, kb = r.standard_normal((B, Hq, nb, D)), r.standard_normal((B, Hkv, nb, D))
    got = o.block_scores(qb, kb)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(nb):
                for j in range(nb):
                    s = 0.0
                    for d in range(D):
                        s += qb[b, h, i, d] * kb[b, g, j, d]
                    assert abs(got[b, h, i, j] - s) <= 1e-14
    # library: einsum over repeat_interleaved KV heads (consecutive query heads share one)
    kt = torch.from_numpy(kb).repeat_interleave(Hq // Hkv, dim=1)
    ref = torch.einsum("bhid,bhjd->bhij", torch.from_numpy(qb), kt).numpy()
    assert np.allclose(got, ref, rtol=0, atol=1e-13)


def check_select_vs_sort(o=O):
    r = rng(3)
    for trial in range(40):
        nb = int(r.integers(1, 70))
        k = int(r.integers(1, nb + 1))
        if trial % 2:   # heavy ties: few distinct values
            S = r.integers(-2, 3, size=(3, 4, nb)).astype(np.float64)
        else:
            S = r.standard_normal((3, 4, nb))
        got = o.select_topk(S, k)
        for row, sel in zip(S.reshape(-1, nb), got.reshape(-1, k)):
            order = np.lexsort((np.arange(nb), -row))[:k]     # score desc, index asc
            assert np.array_equal(sel, np.sort(order))
            assert np.all(np.diff(sel) > 0)


def check_select_special(o=O):
    S = np.zeros((1, 1, 6))
    assert o.select_topk(S, 3).tolist() == [[[0, 1, 2]]]          # all tied: lowest indices
    S = np.array([[[0.0, -0.0, 0.0, -1.0, -0.0]]])
    assert o.select_topk(S, 2).tolist() == [[[0, 1]]]             # -0 ties +0
    S = np.array([[[1.0, 5.0, 3.0, 5.0]]])
    assert o.select_topk(S, 1).tolist() == [[[1]]]
    assert o.select_topk(S, 4).tolist() == [[[0, 1, 2, 3]]]


def check_dense_limit(o=O):
    """topk = nb: the method is dense softmax attention (library SDPA in float64)."""
    B, N, H, D, blk = 1, 64, 2, 16, 8
    q, k, v = rand_qkv(B, N, H, H, D, seed=4)
    nb = N // blk
    idx = o.select(q, k, blk, nb)
    assert np.array_equal(idx, np.broadcast_to(np.arange(nb), (B, H, nb, nb)))
    got = o.attend(q, k, v, idx, blk, 1 / math.sqrt(D))
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3).numpy()
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    assert np.allclose(o.dense_attention(q, k, v, 1 / math.sqrt(D)), ref, rtol=0, atol=1e-12)


def check_bruteforce(o=O):
    """Gathered-block attention equals explicitly masked N x N attention."""
    B, N, H, D, blk = 1, 512, 2, 64, 64      # the tiny workload's shape
    q, k, v = rand_qkv(B, N, H, H, D, seed=5)
    nb = N // blk
    out, idx = o.block_sparse_attention(q, k, v, blk, 0.25)
    assert idx.shape == (B, H, nb, 2)
    ref = o.masked_attention_bruteforce(q, k, v, idx, blk, 1 / math.sqrt(D))
    assert np.max(np.abs(out - ref)) <= 1e-12
    # a sparse result differs from the dense one
    assert np.max(np.abs(out - o.dense_attention(q, k, v, 1 / math.sqrt(D)))) > 1e-3


def check_ties_and_zero(o=O):
    B, N, H, D, blk = 1, 64, 1, 8, 8
    q, k, v = rand_qkv(B, N, H, H, D, seed=6)
    k[:, 5 * blk:6 * blk] = k[:, 2 * blk:3 * blk]             # key block 5 duplicates block 2
    S = o.block_scores(o.pool(q, blk), o.pool(k, blk))
    assert np.array_equal(S[..., 5], S[..., 2])
    for kk in range(1, 8):
        idx = o.select_topk(S, kk)
        for row, sel in zip(S.reshape(-1, 8), idx.reshape(-1, kk)):
            # block 5 can only be chosen when block 2 is chosen too
            assert (5 not in sel) or (2 in sel)
    # q == 0: all scores 0, the lowest k blocks win; output = mean of V over them
    z = np.zeros_like(q)
    out, idx = o.block_sparse_attention(z, k, v, blk, 0.5)
    assert np.all(idx == np.arange(4))
    ref = v[:, :4 * blk].mean(axis=1)                          # [B, H, D]
    assert np.allclose(out, ref[:, None], rtol=0, atol=1e-14)


def check_invariants(o=O):
    B, N, H, D, blk = 2, 96, 2, 16, 8
    q, k, v = rand_qkv(B, N, H, H, D, seed=7)
    scale = 1 / math.sqrt(D)
    out, idx = o.block_sparse_attention(q, k, v, blk, 0.25)
    # V constant => output constant
    c = np.full_like(v, -0.625)
    assert np.allclose(o.attend(q, k, c, idx, blk, scale), -0.625, rtol=0, atol=1e-14)
    # permuting the tokens inside every block (K and V together) changes nothing
    perm = np.concatenate([j * blk + rng(8).permutation(blk) for j in range(N // blk)])
    out_p, idx_p = o.block_sparse_attention(q, k[:, perm], v[:, perm], blk, 0.25)
    assert np.array_equal(idx, idx_p)
    assert np.allclose(out, out_p, rtol=0, atol=1e-13)
    # positive scaling of q keeps the selection
    assert np.array_equal(o.select(3.5 * q, k, blk, 3), o.select(q, k, blk, 3))
    # one-hot-by-block V: the weight of every unselected block is exactly zero
    nb = N // blk
    vb = np.zeros((B, N, H, D))
    for t in range(N):
        vb[:, t, :, t // blk] = 1.0
    w = o.attend(q, k, vb, idx, blk, scale)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                rows = w[b, i * blk:(i + 1) * blk, h, :nb]
                sel = np.zeros(nb, dtype=bool)
                sel[idx[b, h, i]] = True
                assert np.all(rows[:, ~sel] == 0.0)
                assert np.all(rows[:, sel] > 0.0)
                assert np.allclose(rows.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def check_gqa(o=O):
    B, N, Hq, Hkv, D, blk = 1, 64, 4, 2, 8, 8
    q, k, v = rand_qkv(B, N, Hq, Hkv, D, seed=9)
    out, idx = o.block_sparse_attention(q, k, v, blk, 0.5)
    kr = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=2).numpy()
    vr = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=2).numpy()
    out_m, idx_m = o.block_sparse_attention(q, kr, vr, blk, 0.5)
    assert np.array_equal(idx, idx_m)
    assert np.allclose(out, out_m, rtol=0, atol=1e-14)


def check_batched(o=O):
    B, N, Hq, Hkv, D, blk = 2, 64, 4, 2, 8, 8
    q, k, v = rand_qkv(B, N, Hq, Hkv, D, seed=10)
    idx = o.select(q, k, blk, 3)
    a = o.attend(q, k, v, idx, blk, 0.3)
    b = o.attend_batched(q, k, v, idx, blk, 0.3)
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def check_causal_select(o=O):
    """Causal selection [R20] against a full sort of each row's admissible blocks."""
    r = rng(11)
    for k in (1, 3, 7):
        S = np.round(r.standard_normal((2, 3, 9, 9)), 1)       # coarse values: many ties
        idx = o.select_topk_causal(S, k)
        for b in range(2):
            for h in range(3):
                for i in range(9):
                    ki = min(k, i + 1)
                    # stable sort of j < i by descending score, then the own block
                    past = np.lexsort((np.arange(i), -S[b, h, i, :i]))[:ki - 1]
                    want = sorted(past.tolist() + [i]) + [-1] * (k - ki)
                    assert idx[b, h, i].tolist() == want
    assert o.select_topk_causal(np.zeros((1, 4, 4)), 2).tolist() == [[[0, -1], [0, 1], [0, 2],
                                                                       [0, 3]]]


def check_causal_dense_limit(o=O):
    """Causal with topk = nb: every earlier block is kept, the result is causal dense
    attention (library SDPA with is_causal, float64)."""
    B, N, H, D, blk = 1, 64, 2, 16, 8
    q, k, v = rand_qkv(B, N, H, H, D, seed=12)
    nb = N // blk
    idx = o.select(q, k, blk, nb, causal=True)
    got = o.attend(q, k, v, idx, blk, 1 / math.sqrt(D), causal=True)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    ref = ref.permute(0, 2, 1, 3).numpy()
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    assert np.allclose(o.dense_attention(q, k, v, 1 / math.sqrt(D), causal=True), ref,
                       rtol=0, atol=1e-12)


def check_causal_bruteforce(o=O):
    """Causal gathered-block attention equals the explicit N x N mask with u <= t."""
    B, N, Hq, Hkv, D, blk = 1, 512, 4, 2, 32, 64
    q, k, v = rand_qkv(B, N, Hq, Hkv, D, seed=13)
    idx = o.select(q, k, blk, 3, causal=True)
    got = o.attend(q, k, v, idx, blk, 0.2, causal=True)
    ref = o.masked_attention_bruteforce(q, k, v, idx, blk, 0.2, causal=True)
    assert np.max(np.abs(got - ref)) <= 1e-12
    assert np.allclose(o.attend_batched(q, k, v, idx, blk, 0.2, causal=True), got,
                       rtol=0, atol=1e-13)
    # the first token of every sequence sees only itself
    kr = np.repeat(k, Hq // Hkv, axis=2)
    vr = np.repeat(v, Hq // Hkv, axis=2)
    assert np.allclose(got[:, 0], vr[:, 0], rtol=0, atol=1e-14)
    assert kr.shape == q.shape


def check_pool_max(o=O):
    """In-block max pooling [R21] against torch.amax, and its invariances."""
    B, N, H, D, blk = 2, 96, 3, 8, 16
    q, _, _ = rand_qkv(B, N, H, H, D, seed=14)
    got = o.pool_max(q, blk)
    ref = torch.from_numpy(q).reshape(B, N // blk, blk, H, D).amax(dim=2).permute(0, 2, 1, 3)
    assert np.array_equal(got, ref.numpy())
    perm = np.concatenate([j * blk + rng(15).permutation(blk) for j in range(N // blk)])
    assert np.array_equal(o.pool_max(q[:, perm], blk), got)
    assert np.all(got >= o.pool(q, blk))
    a = o.select(q, q[:, :, :1], blk, 2, pooling="max")
    S = o.block_scores(got, o.pool_max(q[:, :, :1], blk))
    assert np.array_equal(a, o.select_topk(S, 2))


def check_group_select(o=O):
    """Group-shared selection [R22]: scores of the summed pooled queries of the group,
    one index set per group; G = 1 is per-head selection."""
    B, N, Hq, Hkv, D, blk = 2, 128, 6, 2, 8, 16
    q, k, _ = rand_qkv(B, N, Hq, Hkv, D, seed=16)
    G = Hq // Hkv
    idx = o.select(q, k, blk, 3, group=True)
    qb, kb = o.pool(q, blk), o.pool(k, blk)
    for b in range(B):
        for g in range(Hkv):
            qsum = sum(qb[b, g * G + j] for j in range(G))          # [nb, D]
            S = qsum @ kb[b, g].T
            want = o.select_topk(S[None], 3)[0]
            for j in range(G):
                assert np.array_equal(idx[b, g * G + j], want)
    q1 = q[:, :, :Hkv]
    assert np.array_equal(o.select(q1, k, blk, 3, group=True), o.select(q1, k, blk, 3))
    ci = o.select(q, k, blk, 3, group=True, causal=True)
    assert np.array_equal(ci[:, 0], ci[:, 1]) and np.all(ci[:, :, 0, 1:] == -1)


def _dense_masked_torch(q, k, v, idx, blk, scale, causal):
    """Masked dense attention in torch float64 (explicit N x N mask), for autograd."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    tb = np.arange(N) // blk
    outs = []
    for b in range(B):
        per_h = []
        for h in range(Hq):
            g = h // (Hq // Hkv)
            M = np.zeros((N, N), dtype=bool)
            for t in range(N):
                M[t] = np.isin(tb, idx[b, h, tb[t]])
                if causal:
                    M[t, t + 1:] = False
            z = scale * (q[b, :, h] @ k[b, :, g].T)
            z = z.masked_fill(~torch.from_numpy(M), float("-inf"))
            per_h.append(torch.softmax(z, dim=1) @ v[b, :, g])
        outs.append(torch.stack(per_h, dim=1))
    return torch.stack(outs, dim=0)


def check_backward_autograd(o=O):
    """Backward against torch autograd through the explicitly masked dense attention,
    with GQA, plain and causal."""
    B, N, Hq, Hkv, D, blk = 2, 192, 4, 2, 16, 32
    q, k, v = rand_qkv(B, N, Hq, Hkv, D, seed=17)
    dout = rng(18).standard_normal(q.shape)
    for causal in (False, True):
        idx = o.select(q, k, blk, 3, causal=causal)
        dq, dk, dv = o.attend_backward(q, k, v, idx, blk, 0.3, dout, causal=causal)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        out = _dense_masked_torch(tq, tk, tv, idx, blk, 0.3, causal)
        (out * torch.from_numpy(dout)).sum().backward()
        for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.max(np.abs(mine - ref.numpy())) <= 1e-12


def check_backward_fd_and_invariants(o=O):
    """Central finite differences of sum(out * dout) on a few entries, and the sums that
    softmax rows fix: sum over keys of dV = sum over queries of dO (per KV head), sum over
    keys of dK = 0."""
    B, N, Hq, Hkv, D, blk = 1, 64, 2, 1, 8, 16
    q, k, v = rand_qkv(B, N, Hq, Hkv, D, seed=19)
    dout = rng(20).standard_normal(q.shape)
    idx = o.select(q, k, blk, 2)
    dq, dk, dv = o.attend_backward(q, k, v, idx, blk, 0.5, dout)
    f = lambda qq, kk, vv: float(np.sum(o.attend(qq, kk, vv, idx, blk, 0.5) * dout))
    eps = 1e-6
    r = rng(21)
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            pos = tuple(int(r.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[pos] += eps
            xm[pos] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (f(*args_p) - f(*args_m)) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-7 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])
    assert np.allclose(dv.sum(axis=1)[:, 0], dout.sum(axis=(1, 2)), rtol=0, atol=1e-12)
    assert np.allclose(dk.sum(axis=1), 0.0, rtol=0, atol=1e-12)


def check_lse(o=O):
    """Log-sum-exp of the masked scores against scipy's logsumexp of the dense masked rows."""
    from scipy.special import logsumexp
    B, N, H, D, blk = 1, 128, 2, 16, 32
    q, k, _ = rand_qkv(B, N, H, H, D, seed=22)
    for causal in (False, True):
        idx = o.select(q, k, blk, 2, causal=causal)
        got = o.attend_lse(q, k, idx, blk, 0.25, causal=causal)
        tb = np.arange(N) // blk
        for h in range(H):
            z = 0.25 * (q[0, :, h] @ k[0, :, h].T)
            for t in range(N):
                keep = np.isin(tb, idx[0, h, tb[t]])
                if causal:
                    keep[t + 1:] = False
                assert abs(got[0, h, t] - logsumexp(z[t][keep])) <= 1e-12


def check_decode(o=O):
    """Decode step [R26]: selection against a full sort over the complete earlier blocks plus
    the own block; with topk covering every block the step is causal dense attention of the
    last token (library SDPA on the prefix); gathered keys equal an explicit mask over the
    cache; a zero query with ties takes the lowest blocks."""
    B, Lmax, Hq, Hkv, D, blk = 3, 256, 4, 2, 16, 32
    r = rng(23)
    qt = r.standard_normal((B, Hq, D))
    kc, vc = r.standard_normal((2, B, Lmax, Hkv, D))
    lens = np.array([256, 97, 33])
    kbar = o.pool(kc, blk)                                       # complete-block means
    for topk in (1, 3, 8):
        idx = o.decode_select(qt, kbar, lens, blk, topk)
        for b in range(B):
            own = (lens[b] - 1) // blk
            kb = min(topk, own + 1)
            for h in range(Hq):
                s = kbar[b, h // 2, :own] @ qt[b, h]
                past = np.lexsort((np.arange(own), -s))[:kb - 1]
                assert idx[b, h].tolist() == sorted(past.tolist() + [own]) + [-1] * (topk - kb)
        got = o.decode_attend(qt, kc, vc, idx, lens, blk, 0.25)
        for b in range(B):
            L = lens[b]
            tb = np.arange(L) // blk
            for h in range(Hq):
                keep = np.isin(tb, idx[b, h])
                z = 0.25 * (kc[b, :L, h // 2] @ qt[b, h])
                z = np.where(keep, z, -np.inf)
                p = np.exp(z - z.max())
                assert np.allclose(got[b, h], p @ vc[b, :L, h // 2] / p.sum(), rtol=0, atol=1e-13)
    idx = o.decode_select(qt, kbar, lens, blk, 8)                # covers every block
    got = o.decode_attend(qt, kc, vc, idx, lens, blk, 0.25)
    for b in range(B):
        L = lens[b]
        for h in range(Hq):
            tq = torch.from_numpy(qt[b, h])[None, None, None]    # [1, 1, 1, D]
            tk = torch.from_numpy(kc[b, :L, h // 2])[None, None]
            tv = torch.from_numpy(vc[b, :L, h // 2])[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.25)
            assert np.allclose(got[b, h], ref[0, 0, 0].numpy(), rtol=0, atol=1e-12)
    z = o.decode_select(np.zeros_like(qt), kbar, lens, blk, 3)
    assert z[0, 0].tolist() == [0, 1, 7] and z[2, 0].tolist() == [0, 1, -1]
    # group choice: a full sort of the summed scores of the KV head's query heads (heads 2g,
    # 2g+1 here), shared by both; with one query head per KV head it is the per-head choice
    for topk in (1, 3, 8):
        idx = o.decode_select(qt, kbar, lens, blk, topk, group=True)
        for b in range(B):
            own = (lens[b] - 1) // blk
            kb = min(topk, own + 1)
            for g in range(2):
                s = kbar[b, g, :own] @ (qt[b, 2 * g] + qt[b, 2 * g + 1])
                past = np.lexsort((np.arange(own), -s))[:kb - 1]
                want = sorted(past.tolist() + [own]) + [-1] * (topk - kb)
                assert idx[b, 2 * g].tolist() == want and idx[b, 2 * g + 1].tolist() == want
    kb1 = o.pool(kc[:, :, :1].repeat(4, axis=2), blk)              # Hkv = Hq = 4
    assert np.array_equal(o.decode_select(qt, kb1, lens, blk, 5, group=True),
                          o.decode_select(qt, kb1, lens, blk, 5))


def check_random_fill(o=O):
    """Random places [R27]: SplitMix64 against its published first outputs for seed 0; per
    row the top k - r blocks, r further distinct blocks, ascending; r = 0 is select_topk;
    the draws are uniform over the remaining blocks (chi-square over many rows)."""
    assert [o.splitmix64(0, n) for n in range(3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                                      0x06C45D188009454F]
    r_ = rng(24)
    S = np.round(r_.standard_normal((2, 3, 10, 40)), 1)
    for k, rr in ((6, 2), (8, 8), (5, 0), (40, 3)):
        idx = o.select_topk_random(S, k, rr, seed=1234)
        top = o.select_topk(S, k - rr) if k > rr else np.zeros(S.shape[:-1] + (0,), dtype=int)
        nrows = int(np.prod(S.shape[:-1]))
        for row_i, row_t in zip(idx.reshape(nrows, k), top.reshape(nrows, k - rr)):
            assert np.all(np.diff(row_i) > 0) and row_i.min() >= 0 and row_i.max() < 40
            assert set(row_t.tolist()) <= set(row_i.tolist())
        if rr == 0:
            assert np.array_equal(idx, o.select_topk(S, k))
    assert not np.array_equal(o.select_topk_random(S, 6, 2, 1), o.select_topk_random(S, 6, 2, 2))
    # uniformity: one random place among 19 others, many rows with equal scores for the rest
    S2 = np.zeros((4000, 20))
    S2[:, 0] = 1.0
    picks = o.select_topk_random(S2, 2, 1, seed=99)[:, 1]
    counts = np.bincount(picks, minlength=20)[1:]
    chi2 = float(((counts - 4000 / 19) ** 2 / (4000 / 19)).sum())
    assert chi2 < 45.0, chi2                     # 18 degrees of freedom: p ~ 5e-4
    # without replacement every 2-subset of the 3 non-top blocks is equally likely
    S3 = np.zeros((6000, 4))
    S3[:, 0] = 1.0
    pairs = o.select_topk_random(S3, 3, 2, seed=7)[:, 1:]
    codes = pairs[:, 0] * 4 + pairs[:, 1]
    counts = np.array([(codes == c).sum() for c in (1 * 4 + 2, 1 * 4 + 3, 2 * 4 + 3)])
    assert counts.sum() == 6000
    chi2 = float(((counts - 2000) ** 2 / 2000).sum())
    assert chi2 < 16.0, (counts, chi2)          # 2 degrees of freedom: p ~ 3e-4


def check_overlap(o=O):
    """Overlapping key blocks [R28]: block ranges against the closed form
    nw = ceil((N - b) / s) + 1 with starts j*s; hand-computed pooled values; stride == block
    reduces to the plain partition; union attention against the explicit token mask, against
    dense attention when every key block is chosen, and against dense attention over one
    contiguous token range when two neighbouring blocks are chosen; the selection finds a
    planted key block that only the overlapping geometry has."""
    assert o.key_block_ranges(8, 4, 3) == [(0, 4), (3, 7), (6, 8)]
    for N, b, s in ((64, 16, 12), (256, 64, 48), (8192, 64, 48), (8192, 128, 96), (128, 64, 32),
                    (192, 64, 40), (64, 64, 64)):
        rg = o.key_block_ranges(N, b, s)
        assert len(rg) == -(-(N - b) // s) + 1
        assert [a for a, _ in rg] == [j * s for j in range(len(rg))]
        assert all(e == min(a + b, N) for a, e in rg) and rg[-1][1] == N
    x = np.arange(8.0).reshape(1, 8, 1, 1)
    assert o.pool_key_blocks(x, 4, 3).ravel().tolist() == [1.5, 4.5, 6.5]
    assert o.pool_key_blocks(x, 4, 3, "max").ravel().tolist() == [3.0, 6.0, 7.0]
    q, k, v = rand_qkv(2, 96, 4, 2, 8, seed=31)
    blk = 16
    assert np.allclose(o.pool_key_blocks(k, blk, blk), o.pool(k, blk), rtol=0, atol=1e-15)
    assert np.array_equal(o.pool_key_blocks(k, blk, blk, "max"), o.pool_max(k, blk))
    assert np.array_equal(o.select(q, k, blk, 3, stride=blk), o.select(q, k, blk, 3))
    idx = o.select(q, k, blk, 3)
    assert np.allclose(o.attend(q, k, v, idx, blk, 0.3, stride=blk),
                       o.attend(q, k, v, idx, blk, 0.3), rtol=0, atol=1e-13)
    stride = 12
    nw = len(o.key_block_ranges(96, blk, stride))              # 8 key blocks for 6 query blocks
    assert nw == 8
    r_ = rng(32)
    idx = np.sort(np.stack([np.stack([np.stack([r_.choice(nw, 3, replace=False) for _ in range(6)])
                                      for _ in range(4)]) for _ in range(2)]), axis=-1)
    got = o.attend(q, k, v, idx, blk, 0.3, stride=stride)
    assert np.allclose(got, o.masked_attention_bruteforce(q, k, v, idx, blk, 0.3, stride=stride),
                       rtol=0, atol=1e-13)
    every = np.broadcast_to(np.arange(nw), (2, 4, 6, nw))
    assert np.allclose(o.attend(q, k, v, every, blk, 0.3, stride=stride),
                       o.dense_attention(q, k, v, 0.3), rtol=0, atol=1e-13)
    pair = np.broadcast_to(np.array([2, 3]), (2, 4, 6, 2))     # tokens [24, 52): one range
    rng_ = slice(2 * stride, 3 * stride + blk)
    ref = o.dense_attention(q, k[:, rng_], v[:, rng_], 0.3)
    assert np.allclose(o.attend(q, k, v, pair, blk, 0.3, stride=stride), ref, rtol=0, atol=1e-13)
    # planted: only the tokens of key block 5 (60..75, across query blocks 3 and 4) point
    # along d = 0, the queries too; block 5 must rank first everywhere
    kp = r_.standard_normal((1, 96, 1, 8)) * 0.01
    kp[0, 60:76, 0, 0] += 1.0
    qp = np.zeros((1, 96, 2, 8))
    qp[..., 0] = 1.0
    top = o.select(qp, kp, blk, 1, stride=stride)
    assert np.all(top == 5), top.ravel()
    top2 = o.select(qp, kp, blk, 2, stride=stride, pooling="max")
    assert np.all(top2 == [4, 5]) or np.all(top2 == [5, 6]), top2[0, 0, 0]


ALL_CHECKS = [check_bf16_widen, check_e4m3, check_widen, check_pool, check_scores, check_select_vs_sort,
              check_select_special, check_dense_limit, check_bruteforce, check_ties_and_zero,
              check_invariants, check_gqa, check_batched, check_causal_select,
              check_causal_dense_limit, check_causal_bruteforce, check_pool_max,
              check_group_select, check_backward_autograd, check_backward_fd_and_invariants,
              check_lse, check_decode, check_random_fill, check_overlap]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()


def test_topk_count_golden():
    path = os.path.join(HERE, "golden", "topk_params.txt")
    n = 0
    for line in open(path, encoding="utf-8"):
        if not line.strip() or line.startswith("#"):
            continue
        N, blk, ratio = line.split()[:3]
        nb = int(N) // int(blk)
        exact = math.floor(fractions.Fraction(ratio) * nb)
        assert O.topk_count(float(ratio), nb) == exact
        n += 1
    assert n >= 5


def test_kth_scores():
    S = np.array([[[3.0, 1.0, 2.0, 2.0]]])
    sk, sk1 = O.kth_scores(S, 2)
    assert sk.item() == 2.0 and sk1.item() == 2.0
    sk, sk1 = O.kth_scores(S, 4)
    assert sk.item() == 1.0 and sk1.item() == -np.inf


def test_rejects():
    with pytest.raises(ValueError):
        O.pool(np.zeros((1, 10, 1, 2)), 4)
    with pytest.raises(ValueError):
        O.select_topk(np.zeros((1, 4)), 0)
    with pytest.raises(ValueError):
        O.select_topk(np.zeros((1, 4)), 5)


# ---------------------------------------------------- planted mistakes (CPU)

def _strict_causal(q, k, v, idx, blk, scale, rows=None, causal=False, stride=None):
    """attend with the causal mask u < t (a key never sees itself): a planted mistake."""
    if not causal:
        return O.attend(q, k, v, idx, blk, scale, rows, stride=stride)
    out = O.attend(q, k, v, idx, blk, scale, rows, causal=True)
    B, N, Hq, D = q.shape
    # recompute rows t > 0 of every block without the diagonal term
    Hkv = k.shape[2]
    for b in range(B):
        for h in range(Hq):
            g = O.kv_head(h, Hq, Hkv)
            for i in range(N // blk):
                tok = np.concatenate([np.arange(j * blk, (j + 1) * blk) for j in idx[b, h, i] if j >= 0])
                for t in range(i * blk, (i + 1) * blk):
                    keys = tok[tok < t]
                    if keys.size == 0:
                        continue
                    z = scale * (k[b, keys, g] @ q[b, t, h])
                    p = np.exp(z - z.max())
                    out[b, t, h] = p @ v[b, keys, g] / p.sum()
    return out


def _backward_no_rowterm(q, k, v, idx, blk, scale, dout, causal=False):
    """attend_backward with dS = P * dP (the rowsum(dO * O) term dropped): a planted mistake."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    dq, dk, dv = (np.zeros(x.shape) for x in (q, k, v))
    for b in range(B):
        for h in range(Hq):
            g = O.kv_head(h, Hq, Hkv)
            for i in range(N // blk):
                rows = slice(i * blk, (i + 1) * blk)
                tok = np.concatenate([np.arange(j * blk, (j + 1) * blk) for j in idx[b, h, i] if j >= 0])
                z = scale * (q[b, rows, h] @ k[b, tok, g].T)
                p = np.exp(z - z.max(axis=1, keepdims=True))
                P = p / p.sum(axis=1, keepdims=True)
                dS = P * (dout[b, rows, h] @ v[b, tok, g].T)
                dq[b, rows, h] = scale * dS @ k[b, tok, g]
                np.add.at(dk[b, :, g], tok, scale * dS.T @ q[b, rows, h])
                np.add.at(dv[b, :, g], tok, P.T @ dout[b, rows, h])
    return dq, dk, dv


def _decode_unforced(q_tok, kbar, lens, blk, topk):
    """decode_select choosing among blocks j <= own by score only: a planted mistake."""
    B, Hq, D = q_tok.shape
    out = np.full((B, Hq, topk), -1, dtype=np.int64)
    for b in range(B):
        own = (int(lens[b]) - 1) // blk
        kb = min(topk, own + 1)
        for h in range(Hq):
            s = kbar[b, h * kbar.shape[1] // Hq, :own + 1] @ q_tok[b, h]
            out[b, h, :kb] = O.select_topk(s[None], kb)[0]
    return out


def _random_with_replacement(S, k, r, seed):
    """select_topk_random drawing from all non-top blocks each time (a block can come twice,
    then the row is padded with the next free block): a planted mistake."""
    nb = S.shape[-1]
    rows = S.reshape(-1, nb)
    out = np.empty((rows.shape[0], k), dtype=np.int64)
    for row in range(rows.shape[0]):
        top = O.select_topk(rows[row][None], k - r)[0].tolist() if k > r else []
        rest = [j for j in range(nb) if j not in set(top)]
        picked = set()
        for p in range(r):
            picked.add(rest[O.splitmix64(seed, row * 65536 + p) % len(rest)])
        extra = [j for j in rest if j not in picked][: r - len(picked)]
        out[row] = sorted(top + sorted(picked) + extra)
    return out.reshape(S.shape[:-1] + (k,))


class Mutant:
    """The oracle module with one function replaced by a wrong version."""

    def __init__(self, **repl):
        self.__dict__.update({k: getattr(O, k) for k in dir(O) if not k.startswith("__")})
        self.__dict__.update(repl)


def _fails(check, mutant):
    try:
        check(mutant)
    except AssertionError:
        return True
    return False


def _rebind(fn, mutant):
    """A copy of oracle function `fn` whose globals come from `mutant`."""
    import types
    g = dict(fn.__globals__)
    g.update({k: v for k, v in mutant.__dict__.items()})
    return types.FunctionType(fn.__code__, g, fn.__name__, fn.__defaults__)


def _mutant(**repl):
    m = Mutant(**repl)
    for name in ("select", "block_sparse_attention", "block_scores", "attend", "attend_batched",
                 "dense_attention", "masked_attention_bruteforce", "select_topk_causal",
                 "decode_select", "decode_attend", "select_topk_random", "pool_key_blocks",
                 "union_tokens"):
        if name not in repl:
            setattr(m, name, _rebind(getattr(O, name), m))
    return m


MUTANTS = {
    "pool_sum_not_mean": dict(pool=lambda x, b: O.pool(x, b) * b),
    "pool_drops_last_token": dict(
        pool=lambda x, b: x.reshape(x.shape[0], -1, b, *x.shape[2:])[:, :, :-1].mean(axis=2)
        .transpose(0, 2, 1, 3)),
    "gqa_modulo_mapping": dict(kv_head=lambda h, Hq, Hkv: h % Hkv),
    "scores_transposed": dict(block_scores=lambda qb, kb: np.swapaxes(O.block_scores(qb, kb), -1, -2)),
    "select_ties_to_higher": dict(
        select_topk=lambda S, k: (S.shape[-1] - 1 - O.select_topk(S[..., ::-1], k))[..., ::-1]),
    "select_smallest": dict(select_topk=lambda S, k: O.select_topk(-S, k)),
    "attend_no_max_shift_sign": dict(
        attend=lambda q, k, v, idx, blk, scale, rows=None, causal=False, stride=None:
        O.attend(q, k, v, idx, blk, -scale, rows, causal, stride)),
    "attend_drops_last_block": dict(
        attend=lambda q, k, v, idx, blk, scale, rows=None, causal=False, stride=None:
        O.attend(q, k, v, idx[..., :-1] if idx.shape[-1] > 1 else idx, blk, scale, rows, causal,
                 stride)),
    "causal_diagonal_not_forced": dict(
        select_topk_causal=lambda S, k: np.stack(
            [np.concatenate([O.select_topk(S[..., i, :i + 1], min(k, i + 1)),
                             np.full(S.shape[:-2] + (k - min(k, i + 1),), -1)], axis=-1)
             for i in range(S.shape[-1])], axis=-2)),
    "causal_mask_excludes_self": dict(
        attend=lambda q, k, v, idx, blk, scale, rows=None, causal=False, stride=None:
        _strict_causal(q, k, v, idx, blk, scale, rows, causal, stride)),
    "pool_max_is_min": dict(pool_max=lambda x, b: -O.pool_max(-x, b)),
    "backward_without_row_term": dict(
        attend_backward=lambda q, k, v, idx, blk, scale, dout, causal=False:
        _backward_no_rowterm(q, k, v, idx, blk, scale, dout, causal)),
    "backward_dk_unscaled": dict(
        attend_backward=lambda q, k, v, idx, blk, scale, dout, causal=False:
        (lambda g: (g[0], g[1] / scale, g[2]))(O.attend_backward(q, k, v, idx, blk, scale, dout, causal))),
    "decode_group_first_head_only": dict(
        decode_select=lambda q, kb, lens, blk, topk, group=False: O.decode_select(
            np.repeat(q[:, ::q.shape[1] // kb.shape[1]], q.shape[1] // kb.shape[1], axis=1)
            if group else q, kb, lens, blk, topk, group=False)),
    "decode_own_block_not_forced": dict(
        decode_select=lambda q, kb, lens, blk, topk, group=False: _decode_unforced(q, kb, lens, blk, topk)),
    "random_fill_with_replacement": dict(
        select_topk_random=lambda S, k, r, seed: _random_with_replacement(S, k, r, seed)),
    "lse_log2": dict(attend_lse=lambda q, k, idx, blk, scale, causal=False:
                     O.attend_lse(q, k, idx, blk, scale, causal) / np.log(2.0)),
    "group_first_head_only": dict(
        group_scores=lambda S, Hkv: S.reshape(S.shape[0], Hkv, -1, *S.shape[2:])[:, :, 0]),
    "e4m3_bias_8": dict(decode_e4m3=lambda c: O.decode_e4m3(c) / 2),
    "widen_divides_by_descale": dict(
        widen=lambda x, dt, d=1.0: O.decode_e4m3(x) / np.float64(d) if dt == "fp8"
        else O.widen(x, dt, d)),
    "widen_ignores_descale": dict(
        widen=lambda x, dt, d=1.0: O.decode_e4m3(x) if dt == "fp8" else O.widen(x, dt, d)),
    "bf16_low_bits": dict(widen_bf16_bits=lambda b: np.asarray(b, dtype=np.uint16).astype(np.float64)),
    "topk_round_not_truncate": dict(topk_count=lambda r, nb: int(round(r * nb))),
    "overlap_short_block_dropped": dict(
        key_block_ranges=lambda N, b, s: [r for r in O.key_block_ranges(N, b, s)
                                          if r[1] - r[0] == b]),
    "overlap_pool_divides_by_block": dict(
        pool_key_blocks=lambda x, b, s, pooling="mean": (
            O.pool_key_blocks(x, b, s, pooling) if pooling != "mean" else np.stack(
                [x[:, a:e].sum(axis=1) / b for a, e in O.key_block_ranges(x.shape[1], b, s)],
                axis=2))),
    "overlap_shared_tokens_twice": dict(
        union_tokens=lambda sel, N, b, s: np.concatenate(
            [np.arange(*O.key_block_ranges(N, b, s)[j]) for j in sel if j >= 0])),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    m = _mutant(**MUTANTS[name])
    caught = [c.__name__ for c in ALL_CHECKS if _fails(c, m)]
    if name == "topk_round_not_truncate":
        # rounding differs from truncation on the pages' own parameters (0.3 * 128 = 38.4 no,
        # 0.15 * 8192 = 1228.8 yes)
        assert m.topk_count(0.15, 8192) != O.topk_count(0.15, 8192)
        return
    assert caught, f"no pin catches mutant {name}"
