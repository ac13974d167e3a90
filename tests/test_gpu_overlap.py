"""Parity of overlapping key blocks (the MSA page's §5.3 overlap remedy, read as key blocks that
start every key_stride tokens, the last one ending at token N) with the fp64 oracle: pooled
keys, the selection over the key blocks, and attention over the union of each row's key
blocks (every token once), through the C ABI's extended entry points.

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
from tests.parity import check_idx, check_out, check_random_rows, fp8_figures, to_f64

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


SEL_SHAPES = [
    # B, N, Hq, Hkv, D, block, key_stride, topk
    (2, 64 * 38, 4, 2, 64, 64, 48, 7),      # ratio 0.25: 51 key blocks, the last of 32 tokens
    (1, 128 * 21, 6, 3, 128, 128, 96, 5),   # ratio 0.25 at block 128: 28, the last of 96
    (1, 64 * 300, 4, 1, 128, 64, 48, 90),   # 400 key blocks (7 lanes of columns), GQA 4
    (1, 64 * 20, 2, 2, 64, 64, 40, 9),      # stride 40: 32 key blocks, the last of 40 tokens
    (1, 128 * 10, 2, 1, 64, 128, 64, 4),    # stride block/2: 19 key blocks, all full
]
OPTIONS = [dict(), dict(pooling="max"), dict(group=True), dict(nrand=2)]


@pytest.mark.parametrize("opts", OPTIONS, ids=lambda o: "-".join(f"{k}={v}" for k, v in o.items()) or "plain")
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("shape", SEL_SHAPES, ids=str)
def test_select_overlap(shape, dtype, opts):
    B, N, Hq, Hkv, D, blk, ks, topk = shape
    say(f"[select overlap] dtype={dtype} shape={shape} opts={opts}")
    nkb = bst.key_blocks(N, blk, ks)
    assert nkb == len(O.key_block_ranges(N, blk, ks))
    q, k, _, _ = syn.iid_inputs(B, N, Hq, Hkv, D, dtype, index=27, device=DEV)
    seed = 0xC0FFEE
    idx, qbar, kbar = bst.select(q, k, blk, topk, key_stride=ks, return_pooled=True, seed=seed,
                                 **opts)
    torch.cuda.synchronize()
    assert idx.shape == (B, Hq, N // blk, topk)
    pooling = opts.get("pooling", "mean")
    qo, ko = stored_values(q), stored_values(k)
    pk = O.pool_key_blocks(ko, blk, ks, pooling)
    pq = (O.pool if pooling == "mean" else O.pool_max)(qo, blk)
    assert np.max(np.abs(kbar.cpu().numpy() - pk)) <= 2e-6 * np.abs(ko).max()
    if not opts.get("group"):
        assert np.max(np.abs(qbar.cpu().numpy() - pq)) <= 2e-6 * np.abs(qo).max()
    S = O.block_scores(pq, pk)                          # [B, Hq, nb, nkb]
    gidx = idx.cpu().numpy()
    if opts.get("group"):
        G = Hq // Hkv
        for j in range(1, G):
            assert np.array_equal(gidx[:, j::G], gidx[:, ::G])
        gidx, S = gidx[:, ::G], O.group_scores(S, Hkv)
    if opts.get("nrand"):
        nrand = opts["nrand"]
        ref = O.select_topk_random(S, topk, nrand, seed)
        rows_g, rows_r = gidx.reshape(-1, topk), ref.reshape(-1, topk)
        rows_s = S.reshape(-1, nkb)
        assert np.all(np.diff(rows_g, axis=1) > 0) and rows_g.min() >= 0 and rows_g.max() < nkb
        sk, sk1 = O.kth_scores(rows_s, topk - nrand)
        clear = (sk - sk1) > 1e-5 * np.maximum(np.abs(sk), np.abs(sk1))
        assert clear.mean() > 0.8
        bad = np.nonzero(clear & ~np.all(rows_g == rows_r, axis=1))[0]
        assert bad.size == 0, f"{bad.size} clear rows differ, first {bad[:5]}"
        amb = np.nonzero(~clear)[0]
        checked = check_random_rows(rows_g, rows_s, topk, nrand, seed, rows=amb)
        say(f"   clear rows {int(clear.sum())}, ambiguous rows checked {checked}")
    else:
        say("  ", check_idx(gidx, S, topk))


FWD_SHAPES = [
    # B, N, Hq, Hkv, D, block, key_stride, topk
    (2, 64 * 38, 4, 2, 64, 64, 48, 7),
    (1, 64 * 30, 2, 1, 128, 64, 48, 12),
    (1, 128 * 21, 6, 3, 128, 128, 96, 5),   # 64-key steps: the skip falls in the first step
    (1, 128 * 12, 2, 1, 64, 128, 64, 6),    # stride block/2: a skipped first step is all -inf
    (1, 128 * 12, 2, 2, 128, 128, 64, 6),
    (2, 64 * 16, 2, 2, 64, 64, 32, 5),
]


def _fwd_case(shape, dtype, idx, index):
    B, N, Hq, Hkv, D, blk, ks, topk = shape
    q, k, v, ds = syn.iid_inputs(B, N, Hq, Hkv, D, dtype, index=index, device=DEV)
    out = bst.forward(q, k, v, idx, descales=ds, key_stride=ks)
    torch.cuda.synchronize()
    qo, ko, vo = (to_f64(x, d) for x, d in zip((q, k, v), ds))
    ref = O.attend(qo, ko, vo, idx.cpu().numpy(), blk, 1 / math.sqrt(D), stride=ks)
    fp8v = (float(np.abs(vo).max()), topk * blk) if dtype == "fp8" else None
    return out.float().cpu().numpy(), ref, fp8v, (qo, ko, vo)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("shape", FWD_SHAPES, ids=str)
def test_forward_overlap_given_rows(shape, dtype):
    """Rows from the seeded set generator: runs of neighbouring key blocks, runs ending at the
    short last block, random sets, descending rows."""
    B, N, Hq, Hkv, D, blk, ks, topk = shape
    if dtype == "fp8" and D != 128:
        pytest.skip("the fp8 kernel is built for D = 128")
    say(f"[forward overlap, given rows] dtype={dtype} shape={shape}")
    nkb = bst.key_blocks(N, blk, ks)
    idx = syn.random_block_sets(B, Hq, N // blk, nkb, topk, index=28, device=DEV)
    got, ref, fp8v, (qo, ko, vo) = _fwd_case(shape, dtype, idx, 28)
    say("   max_abs, rel_l2 =", check_out(got, ref, dtype, fp8_v=fp8v))
    if dtype == "fp8":
        say("   fp8 figures:", fp8_figures(got, ref, *fp8v))
    if dtype != "fp8":
        # negative control: the shared tokens of neighbouring blocks counted twice differ
        twice = np.full_like(ref, np.nan)
        gi = idx.cpu().numpy()
        ranges = O.key_block_ranges(N, blk, ks)
        for b in range(B):
            for h in range(Hq):
                g = O.kv_head(h, Hq, Hkv)
                for i in range(0, N // blk, 3):                  # the run rows
                    tok = np.concatenate([np.arange(*ranges[j]) for j in gi[b, h, i]])
                    z = (qo[b, i * blk:(i + 1) * blk, h] @ ko[b, tok, g].T) / math.sqrt(D)
                    p = np.exp(z - z.max(axis=1, keepdims=True))
                    twice[b, i * blk:(i + 1) * blk, h] = (p @ vo[b, tok, g]) / p.sum(1, keepdims=True)
        rows = ~np.isnan(twice)
        with pytest.raises(AssertionError):
            check_out(got[rows].reshape(-1, D), twice[rows].reshape(-1, D), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("shape", [
    (2, 64 * 38, 4, 2, 128, 64, 48, 7),
    (1, 128 * 21, 6, 3, 128, 128, 96, 5),
    (1, 64 * 40, 4, 4, 128, 64, 40, 20),
], ids=str)
def test_forward_overlap_selected(shape, dtype):
    """The whole path: the selection's rows feed the attention."""
    B, N, Hq, Hkv, D, blk, ks, topk = shape
    say(f"[forward overlap, selected rows] dtype={dtype} shape={shape}")
    q, k, v, ds = syn.iid_inputs(B, N, Hq, Hkv, D, dtype, index=29, device=DEV)
    idx = bst.select(q, k, blk, topk, key_stride=ks)
    out = bst.forward(q, k, v, idx, descales=ds, key_stride=ks)
    torch.cuda.synchronize()
    qo, ko, vo = (to_f64(x, d) for x, d in zip((q, k, v), ds))
    ref = O.attend(qo, ko, vo, idx.cpu().numpy(), blk, 1 / math.sqrt(D), stride=ks)
    fp8v = (float(np.abs(vo).max()), topk * blk) if dtype == "fp8" else None
    say("   max_abs, rel_l2 =", check_out(out.float().cpu().numpy(), ref, dtype, fp8_v=fp8v))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_overlap_every_block_is_dense(dtype):
    """topk = number of key blocks: the union is every token once, i.e. dense attention."""
    B, N, Hq, Hkv, D, blk, ks = 1, 64 * 9, 2, 2, 64, 64, 48
    nkb = bst.key_blocks(N, blk, ks)
    say(f"[overlap dense limit] dtype={dtype} key blocks={nkb}")
    q, k, v, ds = syn.iid_inputs(B, N, Hq, Hkv, D, dtype, index=30, device=DEV)
    idx = bst.select(q, k, blk, nkb, key_stride=ks)
    assert torch.equal(idx.cpu(), torch.arange(nkb, dtype=torch.int32).expand(B, Hq, N // blk, nkb))
    out = bst.forward(q, k, v, idx, key_stride=ks)
    torch.cuda.synchronize()
    dense = O.dense_attention(to_f64(q), to_f64(k), to_f64(v), 1 / math.sqrt(D))
    check_out(out.float().cpu().numpy(), dense, dtype)


@pytest.mark.parametrize("shape", [
    # 1536 key blocks of 128 tokens, K and V of the head above 64 MiB
    (1, 128 * 1152, 2, 1, 128, 128, 96, 9),
], ids=str)
def test_forward_overlap_large_head(shape):
    B, N, Hq, Hkv, D, blk, ks, topk = shape
    assert N * D * 2 * 2 > 64 << 20
    nkb = bst.key_blocks(N, blk, ks)
    say(f"[forward overlap, large head] shape={shape} key blocks={nkb}")
    q, k, v, ds = syn.iid_inputs(B, N, Hq, Hkv, D, "bf16", index=31, device=DEV)
    idx = syn.random_block_sets(B, Hq, N // blk, nkb, topk, index=31, device=DEV)
    out = bst.forward(q, k, v, idx, key_stride=ks)
    torch.cuda.synchronize()
    nb = N // blk
    rows = syn.sample_rows(12, B * Hq * nb, 31) + [0, 1, B * Hq * nb - 1]
    picks = sorted({(r // (Hq * nb), (r // nb) % Hq, r % nb) for r in rows})
    qo, ko, vo = to_f64(q), to_f64(k), to_f64(v)
    ref = O.attend(qo, ko, vo, idx.cpu().numpy(), blk, 1 / math.sqrt(D), rows=picks, stride=ks)
    got = out.float().cpu().numpy()
    for (b, h, i) in picks:
        sl = (b, slice(i * blk, (i + 1) * blk), h)
        check_out(got[sl], ref[sl], "bf16")


def test_overlap_out_of_range_entry_poisons_its_rows():
    """An entry >= the number of key blocks is not read: its query block's output is NaN."""
    B, N, H, D, blk, ks, topk = 1, 64 * 8, 2, 64, 64, 48, 3
    nkb = bst.key_blocks(N, blk, ks)                  # 11 > 8 query blocks
    say(f"[overlap invalid entry] key blocks={nkb}")
    q, k, v, _ = syn.iid_inputs(B, N, H, H, D, "bf16", index=32, device=DEV)
    idx = bst.select(q, k, blk, topk, key_stride=ks)
    good = idx.clone()
    good[0, 0, 2] = torch.tensor([nkb - 3, nkb - 2, nkb - 1], dtype=torch.int32)   # >= nb: valid
    bad = good.clone()
    bad[0, 1, 5, 2] = nkb
    ref = bst.forward(q, k, v, good, key_stride=ks)
    out = bst.forward(q, k, v, bad, key_stride=ks)
    torch.cuda.synchronize()
    o, r = out.float(), ref.float()
    assert not torch.isnan(r).any()
    assert torch.isnan(o[0, 5 * blk:6 * blk, 1]).all()
    mask = torch.ones_like(o, dtype=torch.bool)
    mask[0, 5 * blk:6 * blk, 1] = False
    assert torch.equal(o[mask], r[mask])


def test_overlap_validate_mode(monkeypatch):
    """BSATTN_VALIDATE=1 checks rows against the number of key blocks."""
    B, N, H, D, blk, ks, topk = 1, 64 * 8, 2, 64, 64, 48, 3
    nkb = bst.key_blocks(N, blk, ks)
    say(f"[overlap validate] key blocks={nkb}")
    q, k, v, _ = syn.iid_inputs(B, N, H, H, D, "bf16", index=33, device=DEV)
    idx = bst.select(q, k, blk, topk, key_stride=ks)
    idx[0, 0, 0] = torch.tensor([nkb - 3, nkb - 2, nkb - 1], dtype=torch.int32)
    ref = bst.forward(q, k, v, idx, key_stride=ks)
    monkeypatch.setenv("BSATTN_VALIDATE", "1")
    out = bst.forward(q, k, v, idx, key_stride=ks)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    bad = idx.clone()
    bad[0, 1, 4, 2] = nkb
    with pytest.raises(bst.BsattnError) as e:
        bst.forward(q, k, v, bad, key_stride=ks)
    assert e.value.status == 1 and "1 rows" in str(e.value)
