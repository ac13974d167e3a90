"""Parity of the selection options and the causal variant (through the C ABI's extended
entry points) with the fp64 oracle, on seeded inputs.

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
from tests.parity import (check_idx, check_idx_causal, check_out, check_random_rows,
                          fp8_figures, to_f64)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def stored_values(t):
    """What the selection pools: the stored values (fp8: codes without the descale)."""
    if t.dtype == torch.float8_e4m3fn:
        return O.decode_e4m3(t.view(torch.uint8).cpu().numpy())
    return to_f64(t)


SHAPES = [
    # B, N, Hq, Hkv, D, block, topk
    (2, 64 * 37, 4, 2, 64, 64, 7),       # ragged nb, GQA 2
    (1, 128 * 21, 6, 3, 128, 128, 5),    # block 128, D 128
    (1, 64 * 300, 4, 1, 128, 64, 90),    # nb 300 (5 lanes of columns), GQA 4
]
OPTIONS = [
    dict(causal=True), dict(pooling="max"), dict(group=True),
    dict(causal=True, group=True), dict(causal=True, pooling="max"),
]


@pytest.mark.parametrize("opts", OPTIONS, ids=lambda o: "-".join(f"{k}={v}" for k, v in o.items()))
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_select_options(shape, dtype, opts):
    B, N, Hq, Hkv, D, blk, topk = shape
    say(f"[select options] {opts} dtype={dtype} shape={shape}")
    q, k, _, _ = syn.iid_inputs(B, N, Hq, Hkv, D, dtype, index=21, device=DEV)
    idx = bst.select(q, k, blk, topk, **opts).cpu().numpy()
    qo, ko = stored_values(q), stored_values(k)
    pf = O.pool_max if opts.get("pooling") == "max" else O.pool
    S = O.block_scores(pf(qo, blk), pf(ko, blk))
    G = Hq // Hkv
    if opts.get("group"):
        for j in range(1, G):                      # every head of a group shares the rows
            assert np.array_equal(idx[:, j::G], idx[:, ::G])
        idx, S = idx[:, ::G], O.group_scores(S, Hkv)
    if opts.get("causal"):
        check_idx_causal(idx, S, topk)
    else:
        say("  ", check_idx(idx, S, topk))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("shape", [
    (2, 64 * 37, 4, 2, 128, 64, 7),
    (1, 128 * 21, 6, 3, 128, 128, 5),
    (1, 64 * 12, 2, 2, 128, 64, 12),      # topk = nb: causal dense limit
    (3, 64 * 9, 2, 1, 128, 64, 1),        # topk = 1: own block only
], ids=str)
def test_forward_causal(shape, dtype):
    B, N, Hq, Hkv, D, blk, topk = shape
    say(f"[forward causal] dtype={dtype} shape={shape}")
    q, k, v, ds = syn.iid_inputs(B, N, Hq, Hkv, D, dtype, index=22, device=DEV)
    idx = bst.select(q, k, blk, topk, causal=True)
    out = bst.forward(q, k, v, idx, descales=ds, causal=True)
    torch.cuda.synchronize()
    qo, ko, vo = (to_f64(x, d) for x, d in zip((q, k, v), ds))
    gidx = idx.cpu().numpy()
    ref = O.attend_batched(qo, ko, vo, gidx, blk, 1 / math.sqrt(D), causal=True)
    got = out.float().cpu().numpy()
    fp8v = (float(np.abs(vo).max()), topk * blk) if dtype == "fp8" else None
    say("   max_abs, rel_l2 =", check_out(got, ref, dtype, fp8_v=fp8v))
    if dtype == "fp8":
        say("   fp8 figures:", fp8_figures(got, ref, *fp8v))
    if topk == N // blk:
        dense = O.dense_attention(qo, ko, vo, 1 / math.sqrt(D), causal=True)
        check_out(got, dense, dtype, fp8_v=fp8v)
    # negative control: the same rows without the causal mask differ
    if dtype != "fp8":
        nomask = O.attend_batched(qo, ko, vo, gidx, blk, 1 / math.sqrt(D), causal=False)
        with pytest.raises(AssertionError):
            check_out(got, nomask, dtype)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [
    # K and V of one (batch, KV head) above the 4 MB L2 and 64 MiB: 128-token blocks in
    # 64-key steps with gathered tiles from the last-level cache or HBM, >1024 key blocks
    (1, 128 * 1152, 2, 1, 128, 128, 9),
    (1, 128 * 2112, 1, 1, 64, 128, 6),
], ids=str)
def test_forward_block128_large_heads(shape, causal):
    B, N, Hq, Hkv, D, blk, topk = shape
    assert N * D * 2 * 2 > 64 << 20
    say(f"[block 128, large heads] shape={shape} causal={causal}")
    q, k, v, ds = syn.iid_inputs(B, N, Hq, Hkv, D, "bf16", index=23, device=DEV)
    ws = torch.empty(bst.select_workspace_bytes(B, N, Hq, Hkv, D, blk), dtype=torch.uint8,
                     device=DEV)
    idx = bst.select(q, k, blk, topk, causal=causal, workspace=ws)
    out = bst.forward(q, k, v, idx, causal=causal)
    torch.cuda.synchronize()
    nb = N // blk
    rows = syn.sample_rows(12, B * Hq * nb, 23) + [B * Hq * nb - 1]
    picks = sorted({(r // (Hq * nb), (r // nb) % Hq, r % nb) for r in rows})
    qo, ko, vo = to_f64(q), to_f64(k), to_f64(v)
    gidx = idx.cpu().numpy()
    ref = O.attend(qo, ko, vo, gidx, blk, 1 / math.sqrt(D), rows=picks, causal=causal)
    got = out.float().cpu().numpy()
    for (b, h, i) in picks:
        sl = (b, slice(i * blk, (i + 1) * blk), h)
        check_out(got[sl], ref[sl], "bf16")


def test_causal_out_of_range_entry_poisons_its_rows():
    """A causal row naming a later block is not read: its query block's output is NaN."""
    say("[causal later block]")
    B, N, H, D, blk, topk = 1, 64 * 8, 2, 64, 64, 3
    q, k, v, _ = syn.iid_inputs(B, N, H, H, D, "bf16", index=23, device=DEV)
    idx = bst.select(q, k, blk, topk, causal=True)
    ref = bst.forward(q, k, v, idx, causal=True)
    bad = idx.clone()
    bad[0, 1, 4, 1] = 6                          # block 6 > 4: after the query block
    out = bst.forward(q, k, v, bad, causal=True)
    torch.cuda.synchronize()
    assert torch.isnan(out[0, 4 * blk:5 * blk, 1].float()).all()
    mask = torch.ones_like(out, dtype=torch.bool)
    mask[0, 4 * blk:5 * blk, 1] = False
    assert torch.equal(out[mask], ref[mask])


def test_causal_validate_mode(monkeypatch):
    say("[causal validate]")
    B, N, H, D, blk, topk = 1, 64 * 8, 2, 64, 64, 3
    q, k, v, _ = syn.iid_inputs(B, N, H, H, D, "bf16", index=23, device=DEV)
    idx = bst.select(q, k, blk, topk, causal=True)
    monkeypatch.setenv("BSATTN_VALIDATE", "1")
    bst.forward(q, k, v, idx, causal=True)
    for edit in (lambda t: t.__setitem__((0, 1, 4, 1), 6),      # later block
                 lambda t: t.__setitem__((0, 0, 1, 2), 0)):     # unused place not -1
        bad = idx.clone()
        edit(bad)
        with pytest.raises(bst.BsattnError) as e:
            bst.forward(q, k, v, bad, causal=True)
        assert e.value.status == 1 and "causal" in str(e.value)
    with pytest.raises(bst.BsattnError):                      # causal rows are not full rows
        bst.forward(q, k, v, idx)
    torch.cuda.synchronize()


def test_select_many_blocks_causal():
    """More than 1024 key blocks (score matrix in the workspace), causal and max pooling."""
    B, N, Hq, Hkv, D, blk, topk = 1, 64 * 1152, 2, 1, 64, 64, 200
    say(f"[select many blocks causal] shape={(B, N, Hq, Hkv, D, blk, topk)}")
    q, k, _, _ = syn.iid_inputs(B, N, Hq, Hkv, D, "bf16", index=24, device=DEV)
    qo, ko = to_f64(q), to_f64(k)
    idx = bst.select(q, k, blk, topk, causal=True).cpu().numpy()
    check_idx_causal(idx, O.block_scores(O.pool(qo, blk), O.pool(ko, blk)), topk)
    idx = bst.select(q, k, blk, topk, pooling="max").cpu().numpy()
    say("  ", check_idx(idx, O.block_scores(O.pool_max(qo, blk), O.pool_max(ko, blk)), topk))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 64 * 1152, 4, 2, 64, 64, 40), (2, 128 * 1088, 8, 2, 128, 128, 9)],
                         ids=str)
def test_select_many_blocks_group(shape, dtype, causal):
    """Group-shared selection over more than 1024 key blocks (score matrix per KV head in the
    workspace): the heads of a group share their rows, which follow the index rule under the
    summed scores of the group."""
    B, N, Hq, Hkv, D, blk, topk = shape
    say(f"[select many blocks group] dtype={dtype} shape={shape} causal={causal}")
    q, k, _, _ = syn.iid_inputs(B, N, Hq, Hkv, D, dtype, index=34, device=DEV)
    ws = torch.empty(bst.select_workspace_bytes(B, N, Hq, Hkv, D, blk), dtype=torch.uint8,
                     device=DEV)
    idx = bst.select(q, k, blk, topk, group=True, causal=causal, workspace=ws).cpu().numpy()
    G = Hq // Hkv
    for j in range(1, G):
        assert np.array_equal(idx[:, j::G], idx[:, ::G])
    S = O.group_scores(O.block_scores(O.pool(stored_values(q), blk), O.pool(stored_values(k), blk)),
                       Hkv)
    if causal:
        check_idx_causal(idx[:, ::G], S, topk)
    else:
        say("  ", check_idx(idx[:, ::G], S, topk))


@pytest.mark.parametrize("opts", [{}, dict(causal=True), dict(group=True)],
                         ids=lambda o: "-".join(o) or "plain")
def test_select_mid_range_blocks(opts):
    """nb = 512: the fused kernel at 8 columns per lane, plain, causal and group."""
    B, N, Hq, Hkv, D, blk, topk = 1, 64 * 512, 4, 2, 128, 64, 150
    say(f"[select nb=512] {opts}")
    q, k, _, _ = syn.iid_inputs(B, N, Hq, Hkv, D, "bf16", index=25, device=DEV)
    idx = bst.select(q, k, blk, topk, **opts).cpu().numpy()
    S = O.block_scores(O.pool(to_f64(q), blk), O.pool(to_f64(k), blk))
    if opts.get("group"):
        assert np.array_equal(idx[:, 1::2], idx[:, ::2])
        idx, S = idx[:, ::2], O.group_scores(S, Hkv)
    if opts.get("causal"):
        check_idx_causal(idx, S, topk)
    else:
        say("  ", check_idx(idx, S, topk))


@pytest.mark.parametrize("group", [False, True])
@pytest.mark.parametrize("nrand", [1, 3, 7])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_select_random_places(dtype, nrand, group):
    """Random places: rows whose top topk - nrand is clear under the oracle's scores equal the
    oracle's rows exactly (the draws depend only on the seed, the row and the non-top set);
    every row is ascending, distinct and in range."""
    B, N, Hq, Hkv, D, blk, topk = 2, 64 * 37, 4, 2, 64, 64, 7
    seed = 0x1234_5678_9ABC_DEF0
    say(f"[select random] dtype={dtype} nrand={nrand} group={group}")
    q, k, _, _ = syn.iid_inputs(B, N, Hq, Hkv, D, dtype, index=26, device=DEV)
    idx = bst.select(q, k, blk, topk, group=group, nrand=nrand, seed=seed).cpu().numpy()
    S = O.block_scores(O.pool(stored_values(q), blk), O.pool(stored_values(k), blk))
    if group:
        assert np.array_equal(idx[:, 1::2], idx[:, ::2])
        idx, S = idx[:, ::2], O.group_scores(S, Hkv)
    ref = O.select_topk_random(S, topk, nrand, seed)
    rows_g, rows_r, rows_s = idx.reshape(-1, topk), ref.reshape(-1, topk), S.reshape(-1, S.shape[-1])
    assert np.all(np.diff(rows_g, axis=1) > 0) and rows_g.min() >= 0 and rows_g.max() < N // blk
    kt = topk - nrand
    if kt > 0:
        sk, sk1 = O.kth_scores(rows_s, kt)
        clear = (sk - sk1) > 1e-5 * np.maximum(np.abs(sk), np.abs(sk1))
    else:
        clear = np.ones(rows_s.shape[0], dtype=bool)
    assert clear.mean() > 0.9
    bad = np.nonzero(clear & ~np.all(rows_g == rows_r, axis=1))[0]
    assert bad.size == 0, f"{bad.size} clear rows differ, first {bad[:5]}"
    # the other rows: a valid top part plus exactly the oracle's draws given that part
    amb = np.nonzero(~clear)[0]
    checked = check_random_rows(rows_g, rows_s, topk, nrand, seed, rows=amb)
    say(f"   clear rows {int(clear.sum())}, ambiguous rows checked {checked}")
    # a different seed changes some rows
    other = bst.select(q, k, blk, topk, group=group, nrand=nrand, seed=seed + 1).cpu().numpy()
    assert not np.array_equal(other, bst.select(q, k, blk, topk, group=group, nrand=nrand,
                                                seed=seed).cpu().numpy())
