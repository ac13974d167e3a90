"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on seeded inputs.

Every test here runs on an MI355X; each prints the case it is about to run first.
"""
import math
import sys

import numpy as np
import pytest
import torch

import block_sparse_top_amd as bst
from block_sparse_top_amd import synthetic as syn
import oracle.bsattn_oracle as O
from tests.parity import (check_idx, check_idx_causal, check_out, dtype_name, fp8_figures,
                          out_errors, to_f64, TOL)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make(B, N, Hq, Hkv, D, dtype, index=11):
    q, k, v, ds = syn.iid_inputs(B, N, Hq, Hkv, D, dtype, index=index, device=DEV)
    return q, k, v, ds


def oracle_inputs(q, k, v, ds):
    return to_f64(q, ds[0]), to_f64(k, ds[1]), to_f64(v, ds[2])


SHAPES = [
    # B, N, Hq, Hkv, D, block, topk
    (1, 512, 2, 2, 64, 64, 2),          # the tiny workload's shape
    (2, 64 * 37, 3, 3, 64, 64, 7),      # ragged: nb=37 (not a multiple of 16 rows or 64 lanes)
    (1, 128 * 21, 6, 3, 128, 128, 5),   # GQA group 2, D=128, block 128, ragged tile count
    (2, 64 * 100, 4, 1, 128, 64, 30),   # GQA group 4, D=128, block 64
    (1, 128 * 40, 2, 2, 64, 128, 40),   # topk = nb (dense limit)
    (3, 64 * 9, 2, 2, 64, 64, 1),       # topk = 1
    (1, 64, 1, 1, 64, 64, 1),           # a single block
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("shape", SHAPES[:4], ids=str)
def test_pool_and_select(dtype, shape):
    B, N, Hq, Hkv, D, blk, topk = shape
    say(f"[select] dtype={dtype} shape={shape}")
    q, k, v, ds = make(B, N, Hq, Hkv, D, dtype)
    idx, qbar, kbar = bst.select(q, k, blk, topk, return_pooled=True)
    torch.cuda.synchronize()
    # pooled values: the oracle pools the stored values (fp8: codes without descale)
    qo = to_f64(q) if dtype != "fp8" else O.decode_e4m3(q.view(torch.uint8).cpu().numpy())
    ko = to_f64(k) if dtype != "fp8" else O.decode_e4m3(k.view(torch.uint8).cpu().numpy())
    pq, pk = O.pool(qo, blk), O.pool(ko, blk)
    scale_q = np.abs(qo).max()
    assert np.max(np.abs(qbar.cpu().numpy() - pq)) <= 2e-6 * scale_q
    assert np.max(np.abs(kbar.cpu().numpy() - pk)) <= 2e-6 * np.abs(ko).max()
    S = O.block_scores(pq, pk)
    stats = check_idx(idx.cpu().numpy(), S, topk)
    say("  ", stats)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_forward(dtype, shape):
    B, N, Hq, Hkv, D, blk, topk = shape
    say(f"[forward] dtype={dtype} shape={shape}")
    q, k, v, ds = make(B, N, Hq, Hkv, D, dtype, index=12)
    idx = bst.select(q, k, blk, topk)
    odt = torch.float32 if dtype == "f32" else torch.bfloat16
    out = torch.full((B, N, Hq, D), float("nan"), dtype=odt, device=DEV)   # NaN prefill
    bst.forward(q, k, v, idx, out=out)
    torch.cuda.synchronize()
    qo, ko, vo = oracle_inputs(q, k, v, ds)
    gidx = idx.cpu().numpy()
    check_idx(gidx, O.block_scores(O.pool(qo, blk), O.pool(ko, blk)), topk)
    ref = O.attend_batched(qo, ko, vo, gidx, blk, 1.0 / math.sqrt(D))
    err = check_out(out.float().cpu().numpy(), ref, dtype)
    say("   max_abs, rel_l2 =", err)
    if topk == N // blk:      # dense limit: also equal to dense attention
        dense = O.dense_attention(qo, ko, vo, 1.0 / math.sqrt(D))
        check_out(out.float().cpu().numpy(), dense, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", ["huge_first", "tiny_all", "huge_later"])
@pytest.mark.parametrize("D,blk", [(64, 64), (128, 64), (64, 128)])
def test_extreme_score_ranges(dtype, case, D, blk):
    """Scores far outside exp2's range: the softmax must still be the exact average
    (covers the kernels' reference-maximum paths; the bf16 kernel does such rows a second
    time, with one wave per work-group for (64, 64) and several for the other shapes)."""
    say(f"[extreme] {case} {dtype} D={D} block={blk}")
    B, N, H, topk = 1, 1024, 2, 6
    nb = N // blk
    g = torch.Generator().manual_seed(31)
    q = torch.randn(B, N, H, D, generator=g)
    k = torch.randn(B, N, H, D, generator=g)
    v = torch.randn(B, N, H, D, generator=g)
    if case == "huge_first":
        q *= 60.0                                  # |scale*q.k| in the thousands
    elif case == "tiny_all":
        k += 10.0                                  # every key shares a large component ...
        q = -3.0 + 0.1 * q                         # ... and every query points against it
    else:
        k[:, (nb - 1) * blk:] *= 40.0              # one key block with huge scores
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v = (x.to(tdt).to(DEV) for x in (q, k, v))
    idx = bst.select(q, k, blk, topk)
    if case == "huge_later":                       # make the last block a late member of every row
        idx = torch.tensor([[0, 1, 2, 3, 4, nb - 1]] * (H * nb), dtype=torch.int32,
                           device=DEV).view(B, H, nb, topk)
    out = bst.forward(q, k, v, idx)
    torch.cuda.synchronize()
    qo, ko, vo = to_f64(q), to_f64(k), to_f64(v)
    ref = O.attend(qo, ko, vo, idx.cpu().numpy(), blk, 1 / math.sqrt(D))
    # near one-hot softmax: outputs are O(|v|), so the max-abs bound scales with them
    err = check_out(out.float().cpu().numpy(), ref, dtype, abs_scale=max(1.0, float(np.abs(ref).max())),
                    rel_scale=10.0 if dtype == "f32" else 1.0)
    say("   max_abs, rel_l2 =", err)


@pytest.mark.parametrize("causal", [False, True], ids=["plain", "causal"])
@pytest.mark.parametrize("D,blk", [(64, 64), (128, 128), (64, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_huge_values_do_not_overflow(dtype, D, blk, causal):
    """Values near the top of the float range with scores whose weights stay inside the
    plain pass's range (|scale*q.k| ~ 46, weights ~ 2^46): sum(p * v) overflows fp32 unless the
    weights are referenced to the row maximum. The output must be finite and match the oracle
    (the bf16 kernel redoes such rows with weights <= 1)."""
    say(f"[huge values] {dtype} D={D} block={blk} causal={causal}")
    B, N, H, topk = 1, 1024, 2, 6
    g = torch.Generator().manual_seed(47)
    u = torch.randn(B, 1, H, D, generator=g)
    a = 46.0 * math.sqrt(D) / (1.4426950408889634 * float((u * u).sum(-1).mean()))
    q = a * u + 0.3 * torch.randn(B, N, H, D, generator=g)
    k = u + 0.3 * torch.randn(B, N, H, D, generator=g)
    v = 1e30 * torch.randn(B, N, H, D, generator=g)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v = (x.to(tdt).to(DEV) for x in (q, k, v))
    idx = bst.select(q, k, blk, topk, causal=causal)
    out = bst.forward(q, k, v, idx, causal=causal)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all(), "output overflowed"
    qo, ko, vo = to_f64(q), to_f64(k), to_f64(v)
    ref = O.attend(qo, ko, vo, idx.cpu().numpy(), blk, 1 / math.sqrt(D), causal=causal)
    # the scores themselves are O(300): fp32 dot products carry ~1e-5 relative error there,
    # which moves the near one-hot weights; bounds scaled by the output magnitude
    err = check_out(got, ref, dtype, abs_scale=float(np.abs(ref).max()),
                    rel_scale=10.0 if dtype == "f32" else 1.0)
    say("   max_abs/max|ref|, rel_l2 =", err[0] / float(np.abs(ref).max()), err[1])


@pytest.mark.parametrize("D,blk", [(64, 64), (128, 128)])
def test_flagged_and_plain_rows_in_one_launch(D, blk):
    """Rows whose weights leave the plain pass's range sit next to rows that do not, in one
    launch: the bf16 kernel redoes only the flagged work-groups, and every row still matches
    the oracle (half of the rows read a key block with huge scores, the others do not)."""
    say(f"[mixed rows] D={D} block={blk}")
    B, N, H, topk = 1, 2048, 2, 5
    nb = N // blk
    g = torch.Generator().manual_seed(43)
    q = torch.randn(B, N, H, D, generator=g)
    k = torch.randn(B, N, H, D, generator=g)
    v = torch.randn(B, N, H, D, generator=g)
    k[:, (nb - 1) * blk:] *= 40.0                  # the last key block: huge scores
    q, k, v = (x.to(torch.bfloat16).to(DEV) for x in (q, k, v))
    rows = []
    for r in range(H * nb):                        # even rows hold the huge block, odd ones not
        base = [(r + 3 * e) % (nb - 1) for e in range(topk)]
        base = sorted(set(base))[:topk - 1] if r % 2 == 0 else sorted(set(base))
        if r % 2 == 0:
            base = base + [nb - 1]
        while len(base) < topk:                    # fill to topk distinct blocks below nb - 1
            base = sorted(set(base) | {min(set(range(nb - 1)) - set(base))})
        rows.append(sorted(base))
    idx = torch.tensor(rows, dtype=torch.int32, device=DEV).view(B, H, nb, topk)
    out = bst.forward(q, k, v, idx)
    torch.cuda.synchronize()
    qo, ko, vo = to_f64(q), to_f64(k), to_f64(v)
    ref = O.attend(qo, ko, vo, idx.cpu().numpy(), blk, 1 / math.sqrt(D))
    got = out.float().cpu().numpy()
    err = check_out(got, ref, "bf16", abs_scale=max(1.0, float(np.abs(ref).max())))
    say("   max_abs, rel_l2 =", err)


def test_tiny_workload_end_to_end():
    w = syn.WORKLOADS["tiny_f32"]
    say("[tiny] block_sparse_attention on", w)
    q, k, v, ds, _ = syn.workload_inputs(w, device=DEV)
    out, idx = bst.block_sparse_attention(q, k, v, w.block, w.ratio, return_idx=True)
    torch.cuda.synchronize()
    qo, ko, vo = oracle_inputs(q, k, v, ds)
    ref, ridx = O.block_sparse_attention(qo, ko, vo, w.block, w.ratio)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    check_out(out.cpu().numpy(), ref, "f32")
    bf = O.masked_attention_bruteforce(qo, ko, vo, ridx, w.block, 1 / math.sqrt(w.D))
    check_out(out.cpu().numpy(), bf, "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_exact_ties_lower_index_wins(dtype):
    B, N, H, D, blk = 1, 64 * 40, 2, 64, 64
    say(f"[ties] dtype={dtype}")
    q, k, v, ds = make(B, N, H, H, D, dtype, index=13)
    k = k.clone()
    # duplicate key blocks: 31 <- 3, 17 <- 9, 39 <- 0
    for dst, src in ((31, 3), (17, 9), (39, 0)):
        k[:, dst * blk:(dst + 1) * blk] = k[:, src * blk:(src + 1) * blk]
    for topk in (1, 5, 20, 39):
        idx = bst.select(q, k, blk, topk).cpu().numpy().reshape(-1, topk)
        for row in idx:
            s = set(row.tolist())
            for dst, src in ((31, 3), (17, 9), (39, 0)):
                assert dst not in s or src in s
    # q == 0: every score is 0, the lowest topk blocks are chosen
    z = torch.zeros_like(q)
    idx = bst.select(z, k, blk, 6).cpu().numpy()
    assert np.all(idx == np.arange(6))


def test_zero_query_closed_form():
    B, N, H, D, blk, topk = 1, 64 * 12, 2, 64, 64, 4
    say("[zero q] closed form")
    q, k, v, ds = make(B, N, H, H, D, "bf16", index=14)
    z = torch.zeros_like(q)
    idx = bst.select(z, k, blk, topk)
    out = bst.forward(z, k, v, idx)
    torch.cuda.synchronize()
    assert np.all(idx.cpu().numpy() == np.arange(topk))
    vo = to_f64(v)
    ref = vo[:, :topk * blk].mean(axis=1)[:, None]        # mean of V over blocks 0..topk-1
    check_out(out.float().cpu().numpy(), np.broadcast_to(ref, out.shape), "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_deterministic(dtype):
    say(f"[determinism] {dtype}")
    q, k, v, ds = make(2, 64 * 64, 4, 2, 64, dtype, index=15)
    a_idx = bst.select(q, k, 64, 19)
    a = bst.forward(q, k, v, a_idx)
    b_idx = bst.select(q, k, 64, 19)
    b = bst.forward(q, k, v, b_idx)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx)
    assert torch.equal(a.view(torch.int16) if dtype == "bf16" else a.view(torch.int32),
                       b.view(torch.int16) if dtype == "bf16" else b.view(torch.int32))


def test_invalid_index_poisons_only_its_rows():
    say("[invalid idx]")
    B, N, H, D, blk, topk = 1, 64 * 8, 2, 64, 64, 3
    q, k, v, ds = make(B, N, H, H, D, "bf16", index=16)
    idx = bst.select(q, k, blk, topk)
    bad = idx.clone()
    bad[0, 1, 5, 2] = 1000
    out = bst.forward(q, k, v, bad)
    ref = bst.forward(q, k, v, idx)
    torch.cuda.synchronize()
    o, r = out.float(), ref.float()
    assert torch.isnan(o[0, 5 * blk:6 * blk, 1]).all()
    mask = torch.ones_like(o, dtype=torch.bool)
    mask[0, 5 * blk:6 * blk, 1] = False
    assert torch.equal(o[mask], r[mask])


def test_validate_mode_rejects_bad_rows(monkeypatch):
    """BSATTN_VALIDATE=1: forward checks idx on the GPU (ascending, in range) and returns
    BSATTN_E_INVALID for a bad row; valid rows give the same output as without the check."""
    say("[validate mode]")
    B, N, H, D, blk, topk = 2, 64 * 8, 2, 64, 64, 3
    q, k, v, ds = make(B, N, H, H, D, "bf16", index=16)
    idx = bst.select(q, k, blk, topk)
    ref = bst.forward(q, k, v, idx)
    monkeypatch.setenv("BSATTN_VALIDATE", "1")
    out = bst.forward(q, k, v, idx)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    for name, edit in [("out of range", lambda t: t.__setitem__((1, 1, 5, 2), 8)),
                       ("negative", lambda t: t.__setitem__((0, 0, 0, 0), -1)),
                       ("descending", lambda t: t.__setitem__((0, 1, 3), t[0, 1, 3].flip(0))),
                       ("duplicate", lambda t: t.__setitem__((1, 0, 7, 1), t[1, 0, 7, 0]))]:
        bad = idx.clone()
        edit(bad)
        with pytest.raises(bst.BsattnError) as e:
            bst.forward(q, k, v, bad)
        assert e.value.status == 1 and "1 rows" in str(e.value), (name, str(e.value))
    monkeypatch.delenv("BSATTN_VALIDATE")
    bad = idx.clone()
    bad[0, 1, 3] = bad[0, 1, 3].flip(0)
    bst.forward(q, k, v, bad)                         # unchecked: accepted
    torch.cuda.synchronize()


def test_mutated_indices_fail_parity():
    """Negative control: the output check catches one dropped or swapped block."""
    say("[mutation]")
    B, N, H, D, blk, topk = 1, 64 * 16, 2, 64, 64, 5
    q, k, v, ds = make(B, N, H, H, D, "bf16", index=17)
    idx = bst.select(q, k, blk, topk)
    out = bst.forward(q, k, v, idx).float().cpu().numpy()
    qo, ko, vo = oracle_inputs(q, k, v, ds)
    gidx = idx.cpu().numpy()
    swapped = gidx.copy()
    swapped[0, 0, 3, 1] = next(j for j in range(N // blk) if j not in gidx[0, 0, 3])
    ref_bad = O.attend_batched(qo, ko, vo, swapped, blk, 1 / math.sqrt(D))
    with pytest.raises(AssertionError):
        check_out(out, ref_bad, "bf16")
    dropped = O.attend(qo, ko, vo, gidx[..., :-1], blk, 1 / math.sqrt(D))
    with pytest.raises(AssertionError):
        check_out(out, dropped, "bf16")


def test_empty_batch():
    say("[empty]")
    q = torch.empty(0, 128, 2, 64, dtype=torch.bfloat16, device=DEV)
    idx = bst.select(q, q, 64, 1)
    assert idx.shape == (0, 2, 2, 1)
    out = bst.forward(q, q, q, idx)
    assert out.shape == (0, 128, 2, 64)


@pytest.mark.slow
def test_sparseformer_full_size():
    """The page's benchmark shape at full size: every selection row vs the oracle, and
    sampled query blocks of the output."""
    w = syn.WORKLOADS["sparseformer_n8192_bf16"]
    say("[full size]", w)
    q, k, v, ds, _ = syn.workload_inputs(w, device=DEV)
    topk = O.topk_count(w.ratio, w.nb)
    idx = bst.select(q, k, w.block, topk)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    bst.forward(q, k, v, idx, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    say("  gpu done; oracle selection")
    qo, ko = to_f64(q), to_f64(k)
    S = O.block_scores(O.pool(qo, w.block), O.pool(ko, w.block))
    del qo, ko
    gidx = idx.cpu().numpy()
    stats = check_idx(gidx, S, topk)
    say("  ", stats)
    rows = syn.sample_rows(48, w.B * w.Hq * w.nb, w.index)
    picks = [(r // (w.Hq * w.nb), (r // w.nb) % w.Hq, r % w.nb) for r in rows]
    bsel = sorted({b for b, _, _ in picks})
    for b in bsel:
        qb, kb, vb = (to_f64(x[b:b + 1]) for x in (q, k, v))
        mine = [(0, h, i) for bb, h, i in picks if bb == b]
        ref = O.attend(qb, kb, vb, gidx[b:b + 1], w.block, 1 / math.sqrt(w.D), rows=mine)
        got = out[b:b + 1].float().cpu().numpy()
        for (_, h, i) in mine:
            sl = (0, slice(i * w.block, (i + 1) * w.block), h)
            check_out(got[sl], ref[sl], "bf16")
    say("  sampled", len(picks), "query blocks ok")


@pytest.mark.parametrize("shape", [
    # B, N, Hq, Hkv, D, block, topk: more than 1024 key blocks (score matrix in the workspace)
    (1, 64 * 2048, 4, 2, 64, 64, 300),
    (1, 128 * 1088, 2, 1, 128, 128, 163),
])
def test_select_many_blocks(shape):
    B, N, Hq, Hkv, D, blk, topk = shape
    say(f"[select many blocks] shape={shape}")
    q, k, v, ds = make(B, N, Hq, Hkv, D, "bf16", index=18)
    del v
    idx, qbar, kbar = bst.select(q, k, blk, topk, return_pooled=True)
    torch.cuda.synchronize()
    qo, ko = to_f64(q), to_f64(k)
    pq, pk = O.pool(qo, blk), O.pool(ko, blk)
    assert np.max(np.abs(qbar.cpu().numpy() - pq)) <= 2e-6 * np.abs(qo).max()
    assert np.max(np.abs(kbar.cpu().numpy() - pk)) <= 2e-6 * np.abs(ko).max()
    stats = check_idx(idx.cpu().numpy(), O.block_scores(pq, pk), topk)
    say("  ", stats)


@pytest.mark.parametrize("dtype", ["f32", "fp8"])
def test_select_many_blocks_dtypes(dtype):
    """More than 1024 key blocks with fp32 and fp8 inputs: both sides pooled by the pool
    kernel (fp8: codes without the descale), the score matrix and the per-row top-k."""
    B, N, Hq, Hkv, D, blk, topk = 1, 64 * 1088, 4, 2, 128, 64, 250
    say(f"[select many blocks] dtype={dtype} shape={(B, N, Hq, Hkv, D, blk, topk)}")
    q, k, _, _ = make(B, N, Hq, Hkv, D, dtype, index=21)
    idx, qbar, kbar = bst.select(q, k, blk, topk, return_pooled=True)
    torch.cuda.synchronize()
    qo = to_f64(q) if dtype != "fp8" else O.decode_e4m3(q.view(torch.uint8).cpu().numpy())
    ko = to_f64(k) if dtype != "fp8" else O.decode_e4m3(k.view(torch.uint8).cpu().numpy())
    pq, pk = O.pool(qo, blk), O.pool(ko, blk)
    assert np.max(np.abs(qbar.cpu().numpy() - pq)) <= 2e-6 * np.abs(qo).max()
    assert np.max(np.abs(kbar.cpu().numpy() - pk)) <= 2e-6 * np.abs(ko).max()
    say("  ", check_idx(idx.cpu().numpy(), O.block_scores(pq, pk), topk))


@pytest.mark.parametrize("shape", [
    # B, N, Hq, Hkv, D, block: more than 1024 key blocks (the score matrix stays in the workspace)
    (1, 64 * 2048, 2, 1, 64, 64),
    (1, 128 * 1088, 2, 2, 128, 128),
])
def test_score_matrix_fp32_accuracy(shape):
    """The score matrix of the many-block selection is formed on the bf16 MFMA from three-part
    bf16 splits of the pooled values (fp32 accuracy): checked on the hardware against the fp64
    product of the same pooled rows (the GPU's own, read from the workspace), relative to
    sum_d |qbar_d kbar_d|. An fp32 matrix product reaches about 2e-7 on such rows; a two-part
    split would leave terms near 2^-16 = 1.5e-5."""
    B, N, Hq, Hkv, D, blk = shape
    nb = N // blk
    say(f"[score matrix accuracy] shape={shape}")
    q, k, _, _ = make(B, N, Hq, Hkv, D, "bf16", index=20)
    ws = torch.empty(bst.select_workspace_bytes(B, N, Hq, Hkv, D, blk), dtype=torch.uint8, device=DEV)
    idx, qbar, kbar = bst.select(q, k, blk, 16, return_pooled=True, workspace=ws)
    torch.cuda.synchronize()
    kb_bytes = (B * Hkv * nb * D * 4 + 255) // 256 * 256
    qb_bytes = (B * Hq * nb * D * 4 + 255) // 256 * 256
    S = ws[qb_bytes + kb_bytes: qb_bytes + kb_bytes + B * Hq * nb * nb * 4].view(torch.float32)
    S = S.view(B, Hq, nb, nb).cpu().numpy().astype(np.float64)
    qb = qbar.cpu().numpy().astype(np.float64)
    kb = kbar.cpu().numpy().astype(np.float64)
    G = Hq // Hkv
    worst = 0.0
    for b in range(B):
        for h in range(Hq):
            exact = qb[b, h] @ kb[b, h // G].T
            mag = np.abs(qb[b, h]) @ np.abs(kb[b, h // G]).T
            worst = max(worst, float(np.max(np.abs(S[b, h] - exact) / mag)))
    say("   max |S - exact| / sum|q k| =", worst)
    assert worst <= 1e-6


def test_select_many_blocks_ties_and_outliers():
    """The per-row selection over more than 1024 key blocks on rows that stress its threshold
    search: exact ties (duplicated key blocks: the lower index wins), a zero query (every score
    equal), one key block far above the rest (the others' scores crowd into one value bucket),
    k = 1 and k = nb, plain and causal."""
    B, N, H, D, blk = 1, 64 * 1152, 2, 64, 64
    nb = N // blk
    say(f"[select many blocks: ties and outliers] nb={nb}")
    q, k, v, ds = make(B, N, H, H, D, "bf16", index=19)
    del v
    k = k.clone()
    dups = ((1100, 3), (517, 9), (1151, 0), (600, 599))
    for dst, src in dups:
        k[:, dst * blk:(dst + 1) * blk] = k[:, src * blk:(src + 1) * blk]
    qo, ko = to_f64(q), to_f64(k)
    S = O.block_scores(O.pool(qo, blk), O.pool(ko, blk))
    for topk in (1, 173, 576, nb):
        idx = bst.select(q, k, blk, topk).cpu().numpy()
        say("   topk", topk, check_idx(idx, S, topk))
        for row in idx.reshape(-1, topk):
            chosen = set(row.tolist())
            for dst, src in dups:
                assert dst not in chosen or src in chosen
    idx = bst.select(q, k, blk, 300, causal=True).cpu().numpy()
    check_idx_causal(idx, S, 300)
    # zero query: every score is 0, the lowest blocks are chosen
    idx = bst.select(torch.zeros_like(q), k, blk, 200).cpu().numpy()
    assert np.all(idx == np.arange(200))
    idx = bst.select(torch.zeros_like(q), k, blk, 200, causal=True).cpu().numpy()
    for i in range(nb):
        n = min(200, i + 1)
        assert np.all(idx[:, :, i, :n - 1] == np.arange(n - 1)) and np.all(idx[:, :, i, n - 1] == i)
        assert np.all(idx[:, :, i, n:] == -1)
    # one key block far above the rest
    k2 = k.clone()
    k2[:, 700 * blk:701 * blk] *= 3.0e4
    S2 = O.block_scores(O.pool(qo, blk), O.pool(to_f64(k2), blk))
    idx = bst.select(q, k2, blk, 150).cpu().numpy()
    say("   outlier", check_idx(idx, S2, 150))


def test_planted_workload_sampled():
    """The planted-structure workload at full size: every selection row vs the oracle
    (the planted blocks are recovered statistically, not asserted), sampled outputs."""
    w = syn.WORKLOADS["planted_n32768_bf16"]
    say("[planted]", w)
    q, k, v, ds, extra = syn.workload_inputs(w, device=DEV)
    topk = O.topk_count(w.ratio, w.nb)
    idx = bst.select(q, k, w.block, topk)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    bst.forward(q, k, v, idx, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    qo, ko = to_f64(q), to_f64(k)
    gidx = idx.cpu().numpy()
    stats = check_idx(gidx, O.block_scores(O.pool(qo, w.block), O.pool(ko, w.block)), topk)
    planted = extra["planted"].cpu().numpy()
    hit = np.mean([len(set(a) & set(b)) / topk for a, b in
                   zip(gidx.reshape(-1, topk), planted.reshape(-1, topk))])
    say("  ", stats, "planted recovery", round(float(hit), 3))
    rows = syn.sample_rows(24, w.B * w.Hq * w.nb, w.index)
    picks = [(r // (w.Hq * w.nb), (r // w.nb) % w.Hq, r % w.nb) for r in rows]
    vo = to_f64(v)
    ref = O.attend(qo, ko, vo, gidx, w.block, 1 / math.sqrt(w.D), rows=picks)
    got = out.float().cpu().numpy()
    for (b, h, i) in picks:
        sl = (b, slice(i * w.block, (i + 1) * w.block), h)
        check_out(got[sl], ref[sl], "bf16")


@pytest.mark.slow
def test_long_context_gqa_sampled():
    """1M tokens, 32 query / 8 KV heads, 8192 key blocks: sampled rows of the selection and
    of the output against the oracle (which pools all keys of the sampled heads)."""
    w = syn.WORKLOADS["longctx_gqa_n1m_bf16"]
    say("[long context]", w)
    q, k, v, ds, _ = syn.workload_inputs(w, device=DEV)
    topk = O.topk_count(w.ratio, w.nb)
    ws = torch.empty(bst.select_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.block),
                     dtype=torch.uint8, device=DEV)
    idx = bst.select(q, k, w.block, topk, workspace=ws)
    del ws
    out = bst.forward(q, k, v, idx)
    torch.cuda.synchronize()
    say("  gpu done")
    G = w.Hq // w.Hkv
    rows = syn.sample_rows(64, w.Hq * w.nb, w.index)      # 64 seeded (head, query block) rows
    picks = [(0, r // w.nb, r % w.nb) for r in rows]
    tally = {"clear": 0, "ambiguous": 0}
    gidx = idx.cpu().numpy()
    qfull = np.zeros((1, w.N, 1, w.D))
    for g in sorted({h // G for _, h, _ in picks}):
        kg = to_f64(k[:, :, g:g + 1])                                  # [1, N, 1, D]
        vg = to_f64(v[:, :, g:g + 1])
        kbar = O.pool(kg, w.block)[0, 0]                               # [nb, D]
        for (_, h, i) in [p for p in picks if p[1] // G == g]:
            blk = slice(i * w.block, (i + 1) * w.block)
            qb = to_f64(q[:, blk, h:h + 1])                            # [1, block, 1, D]
            s = O.pool(qb, w.block)[0, 0, 0] @ kbar.T                  # [nb]
            st = check_idx(gidx[0, h, i][None], s[None], topk)
            tally["clear"] += st["clear"]
            tally["ambiguous"] += st["ambiguous"]
            qfull[:, blk] = qb
            ref = O.attend(qfull, kg, vg, gidx[:, h:h + 1], w.block, 1 / math.sqrt(w.D),
                           rows=[(0, 0, i)])
            qfull[:, blk] = 0.0
            check_out(out[0, blk, h].float().cpu().numpy(), ref[0, blk, 0], "bf16")
        say(f"  kv head {g} ok")
    say("  64 sampled rows:", tally)
    assert tally["clear"] + tally["ambiguous"] == 64


@pytest.mark.slow
def test_long_context_causal_selection_sampled():
    """1M tokens, 32 query / 8 KV heads, causal selection over 8192 key blocks (the score
    product forms only the tiles on and below the diagonal; rows with i + 1 <= k skip the
    search): 64 seeded sampled rows hold min(k, i+1) blocks, the own block last, then -1, and
    their other blocks follow the index rule under the oracle's scores of the blocks j < i."""
    w = syn.WORKLOADS["longctx_gqa_n1m_bf16"]
    say("[long context causal selection]", w)
    q, k, _, _, _ = syn.workload_inputs(w, device=DEV)
    topk = O.topk_count(w.ratio, w.nb)
    ws = torch.empty(bst.select_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.block),
                     dtype=torch.uint8, device=DEV)
    idx = bst.select(q, k, w.block, topk, causal=True, workspace=ws).cpu().numpy()
    del ws
    say("  gpu done")
    G = w.Hq // w.Hkv
    rows = syn.sample_rows(64, w.Hq * w.nb, w.index + 1)  # 64 seeded (head, query block) rows
    picks = [(r // w.nb, r % w.nb) for r in rows]
    n_short = 0
    for g in sorted({h // G for h, _ in picks}):
        kbar = O.pool(to_f64(k[:, :, g:g + 1]), w.block)[0, 0]        # [nb, D]
        for h, i in [p for p in picks if p[0] // G == g]:
            qb = to_f64(q[:, i * w.block:(i + 1) * w.block, h:h + 1])  # [1, block, 1, D]
            s = O.pool(qb, w.block)[0, 0, 0] @ kbar.T                 # [nb]
            row = idx[0, h, i]
            ki = min(topk, i + 1)
            assert np.all(row[ki:] == -1), f"head {h} row {i}: unused places not -1"
            assert row[ki - 1] == i, f"head {h} row {i}: own block not last"
            if ki > 1:
                check_idx(np.ascontiguousarray(row[:ki - 1])[None], s[None, :i], ki - 1)
            n_short += i + 1 <= topk
        say(f"  kv head {g} ok")
    say(f"  64 sampled causal rows, {n_short} of them with i + 1 <= k")


FP8_SHAPES = [
    # B, N, Hq, Hkv, D, block, topk (the fp8 kernel is built for D = 128)
    (1, 64 * 8, 2, 2, 128, 64, 8),          # topk = nb: dense limit
    (2, 64 * 37, 4, 2, 128, 64, 11),        # ragged nb, GQA 2
    (1, 128 * 21, 6, 3, 128, 128, 5),       # block 128
    (1, 64 * 40, 2, 2, 128, 64, 1),         # topk = 1
]


@pytest.mark.parametrize("shape", FP8_SHAPES, ids=str)
def test_forward_fp8(shape):
    B, N, Hq, Hkv, D, blk, topk = shape
    say(f"[forward fp8] shape={shape}")
    q, k, v, ds = make(B, N, Hq, Hkv, D, "fp8", index=19)
    idx = bst.select(q, k, blk, topk)
    out = torch.full((B, N, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    bst.forward(q, k, v, idx, descales=ds, out=out)
    torch.cuda.synchronize()
    qo, ko, vo = oracle_inputs(q, k, v, ds)
    gidx = idx.cpu().numpy()
    check_idx(gidx, O.block_scores(O.pool(qo, blk), O.pool(ko, blk)), topk)
    ref = O.attend_batched(qo, ko, vo, gidx, blk, 1.0 / math.sqrt(D))
    vmax = float(np.abs(vo).max())
    got = out.float().cpu().numpy()
    err = check_out(got, ref, "fp8", fp8_v=(vmax, topk * blk))
    say("   fp8 figures:", fp8_figures(got, ref, vmax, topk * blk))
    if topk == 1 or topk == N // blk:
        return
    # negative control at this bound: one dropped block of a few is caught
    few = idx[..., :3].contiguous() if topk > 3 else idx
    out3 = bst.forward(q, k, v, few, descales=ds).float().cpu().numpy()
    g3 = few.cpu().numpy()
    dropped = O.attend_batched(qo, ko, vo, g3[..., :-1], blk, 1.0 / math.sqrt(D))
    with pytest.raises(AssertionError):
        check_out(out3, dropped, "fp8", fp8_v=(vmax, 2 * blk))


def test_fp8_workload_sampled():
    """The fp8 workload at full size: every selection row vs the oracle (pooled per batch
    element), sampled query blocks of the output."""
    w = syn.WORKLOADS["fp8_n65536"]
    say("[fp8 workload]", w)
    q, k, v, ds, _ = syn.workload_inputs(w, device=DEV)
    topk = O.topk_count(w.ratio, w.nb)
    idx = bst.select(q, k, w.block, topk)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    bst.forward(q, k, v, idx, descales=ds, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    gidx = idx.cpu().numpy()
    for b in range(w.B):
        qb, kb = to_f64(q[b:b + 1], ds[0]), to_f64(k[b:b + 1], ds[1])
        check_idx(gidx[b:b + 1], O.block_scores(O.pool(qb, w.block), O.pool(kb, w.block)), topk)
    say("  selection ok")
    rows = syn.sample_rows(16, w.B * w.Hq * w.nb, w.index)
    picks = [(r // (w.Hq * w.nb), (r // w.nb) % w.Hq, r % w.nb) for r in rows]
    for b in sorted({p[0] for p in picks}):
        qb, kb, vb = (to_f64(x[b:b + 1], d) for x, d in zip((q, k, v), ds))
        mine = [(0, h, i) for bb, h, i in picks if bb == b]
        ref = O.attend(qb, kb, vb, gidx[b:b + 1], w.block, 1 / math.sqrt(w.D), rows=mine)
        got = out[b:b + 1].float().cpu().numpy()
        vmax = float(np.abs(vb).max())
        for (_, h, i) in mine:
            sl = (0, slice(i * w.block, (i + 1) * w.block), h)
            check_out(got[sl], ref[sl], "fp8", fp8_v=(vmax, topk * w.block))
            say("   fp8 figures", (b, h, i), fp8_figures(got[sl], ref[sl], vmax, topk * w.block))
    say("  sampled outputs ok")
