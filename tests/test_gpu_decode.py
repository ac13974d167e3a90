"""Parity of the decode step (pooled-key cache upkeep, block choice, attention) through the
C ABI with the fp64 oracle, on seeded caches.

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
from tests.parity import check_idx, check_out, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def caches(B, Lmax, Hq, Hkv, D, index):
    q, k, v, _ = syn.iid_inputs(B, Lmax, Hq, Hkv, D, "bf16", index=index, device=DEV)
    return q[:, 0].contiguous(), k, v                      # one query row per sequence


def check_decode_idx(gidx, qo, kbar_o, lens, blk, topk):
    """Own block last, -1 after min(topk, own+1) places, the rest under the index rule
    against the oracle's scores of the complete earlier blocks."""
    B, Hq, _ = gidx.shape
    Hkv = kbar_o.shape[1]
    for b in range(B):
        own = (int(lens[b]) - 1) // blk
        kb = min(topk, own + 1)
        assert np.all(gidx[b, :, kb - 1] == own) and np.all(gidx[b, :, kb:] == -1)
        if kb > 1:
            S = np.stack([kbar_o[b, h // (Hq // Hkv), :own] @ qo[b, h] for h in range(Hq)])
            check_idx(np.ascontiguousarray(gidx[b, :, :kb - 1]), S, kb - 1)


CASES = [
    # B, Lmax, Hq, Hkv, D, block, topk, lens
    (4, 64 * 20, 4, 2, 64, 64, 5, [1280, 97, 1, 64 * 7]),
    (3, 128 * 12, 8, 2, 128, 128, 3, [1536, 1000, 129]),
    (2, 64 * 40, 4, 4, 128, 64, 1, [2560, 65]),
    (2, 64 * 16, 2, 1, 64, 64, 16, [1024, 700]),          # topk covers every block
    # more key blocks: 4, 16 and 32 columns per lane (4 waves per head), then 64 and 128
    # (one wave per head)
    (2, 64 * 200, 4, 2, 64, 64, 20, [12800, 5000]),
    (2, 64 * 1000, 8, 2, 128, 64, 76, [64000, 33333]),
    (1, 64 * 2000, 4, 2, 64, 64, 50, [128000]),
    (1, 64 * 3000, 2, 1, 64, 64, 30, [192000]),
    (1, 64 * 8192, 2, 1, 64, 64, 40, [524288]),
    # many sequences: 128 x 32 heads = 4096 one-wave heads, where the launch gives each head
    # one split (the split rule's lower clamp)
    (128, 64 * 8, 32, 8, 64, 64, 3, [1 + (37 * i) % 512 for i in range(127)] + [512]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: str(c[:7]))
def test_decode(case):
    B, Lmax, Hq, Hkv, D, blk, topk, lens_l = case
    say(f"[decode] {case}")
    q, kc, vc = caches(B, Lmax, Hq, Hkv, D, index=41)
    lens = torch.tensor(lens_l, dtype=torch.int32, device=DEV)
    kbar = torch.full((B, Hkv, D, Lmax // blk), float("nan"), dtype=torch.float32, device=DEV)
    bst.decode_pool(kc, lens, kbar, blk)
    out, idx = bst.decode(q, kc, vc, kbar, lens, blk, topk)
    torch.cuda.synchronize()
    qo, ko, vo = to_f64(q), to_f64(kc), to_f64(vc)
    kbar_o = O.pool(ko, blk)
    kg = kbar.cpu().numpy().transpose(0, 1, 3, 2)           # -> [B, Hkv, nb, D]
    for b in range(B):                                       # complete blocks only
        nc = lens_l[b] // blk
        assert np.max(np.abs(kg[b, :, :nc] - kbar_o[b, :, :nc]), initial=0.0) <= 2e-6 * np.abs(ko).max()
    gidx = idx.cpu().numpy()
    check_decode_idx(gidx, qo, kbar_o, lens_l, blk, topk)
    ref = O.decode_attend(qo, ko, vo, gidx, lens_l, blk, 1 / math.sqrt(D))
    say("   max_abs, rel_l2 =", check_out(out.float().cpu().numpy(), ref, "bf16"))
    if topk >= Lmax // blk:                                  # dense limit of the last token
        dense = O.decode_attend(qo, ko, vo, np.tile(np.arange(Lmax // blk), (B, Hq, 1)),
                                lens_l, blk, 1 / math.sqrt(D))
        check_out(out.float().cpu().numpy(), dense, "bf16")


GROUP_CASES = [
    # B, Lmax, Hq, Hkv, D, block, topk, lens (GQA 2 to 16, every selection-kernel form)
    (4, 64 * 20, 4, 2, 64, 64, 5, [1280, 97, 1, 64 * 7]),
    (3, 128 * 12, 8, 2, 128, 128, 3, [1536, 1000, 129]),
    (2, 64 * 1000, 8, 2, 128, 64, 76, [64000, 33333]),
    (1, 64 * 3000, 8, 1, 64, 64, 30, [192000]),
    (2, 64 * 40, 16, 1, 64, 64, 9, [2560, 700]),     # G = 16: the largest group of one work-group
    # the tile transfers of the group kernel: 16 per wave per tile (more than its fixed waits
    # name: the wait-for-all form), and G = 3 (the tile's 8 transfers do not split evenly, the
    # last wave repeats one)
    (2, 128 * 10, 4, 2, 128, 128, 4, [1280, 300]),
    (2, 64 * 30, 6, 2, 64, 64, 6, [1920, 555]),
    # 128 sequences x 8 KV heads = 1024 four-wave work-groups, one split each
    (128, 64 * 8, 32, 8, 64, 64, 3, [1 + (37 * i) % 512 for i in range(127)] + [512]),
]


@pytest.mark.parametrize("case", GROUP_CASES, ids=lambda c: str(c[:7]))
def test_decode_group(case):
    """Group-shared decode selection: the query heads of a KV head share one row, which
    follows the index rule under the sum of their scores; outputs against the oracle."""
    B, Lmax, Hq, Hkv, D, blk, topk, lens_l = case
    say(f"[decode group] {case}")
    q, kc, vc = caches(B, Lmax, Hq, Hkv, D, index=42)
    lens = torch.tensor(lens_l, dtype=torch.int32, device=DEV)
    kbar = torch.empty((B, Hkv, D, Lmax // blk), dtype=torch.float32, device=DEV)
    bst.decode_pool(kc, lens, kbar, blk)
    out, idx = bst.decode(q, kc, vc, kbar, lens, blk, topk, group=True)
    torch.cuda.synchronize()
    qo, ko, vo = to_f64(q), to_f64(kc), to_f64(vc)
    kbar_o = O.pool(ko, blk)
    gidx = idx.cpu().numpy()
    G = Hq // Hkv
    for j in range(1, G):
        assert np.array_equal(gidx[:, j::G], gidx[:, ::G])
    qsum = qo.reshape(B, Hkv, G, D).sum(axis=2)              # [B, Hkv, D]
    check_decode_idx(gidx[:, ::G], qsum, kbar_o, lens_l, blk, topk)
    ref = O.decode_attend(qo, ko, vo, gidx, lens_l, blk, 1 / math.sqrt(D))
    check_out(out.float().cpu().numpy(), ref, "bf16")
    # the oracle's own group choice agrees on the rows where the order is clear
    want = O.decode_select(qo, kbar_o, lens_l, blk, topk, group=True)
    agree = float(np.mean(np.all(want == gidx, axis=-1)))
    say(f"   rows equal to the oracle's group choice: {agree:.3f}")
    assert agree > 0.9


def test_decode_incremental_pool_and_invalid_length():
    """Appending tokens block by block keeps kbar equal to a full pooling; a sequence with an
    invalid length gets idx -1 and NaN output, the others are unaffected."""
    B, Lmax, Hq, Hkv, D, blk = 3, 64 * 10, 4, 2, 64, 64
    say("[decode incremental]")
    q, kc, vc = caches(B, Lmax, Hq, Hkv, D, index=42)
    kbar = torch.zeros((B, Hkv, D, Lmax // blk), dtype=torch.float32, device=DEV)
    lens_seq = [[1, 5, 64], [63, 64, 65], [128, 200, 640], [640, 400, 640]]
    prev = torch.zeros(B, dtype=torch.int32, device=DEV)
    for ls in lens_seq[:3]:
        cur = torch.tensor(ls, dtype=torch.int32, device=DEV)
        bst.decode_pool(kc, cur, kbar, blk, lens_old=prev)
        prev = cur
    full = torch.zeros_like(kbar)
    bst.decode_pool(kc, prev, full, blk)
    torch.cuda.synchronize()
    for b in range(B):
        nc = int(prev[b]) // blk
        assert torch.equal(kbar[b, :, :, :nc], full[b, :, :, :nc])
    lens = torch.tensor([640, 0, 300], dtype=torch.int32, device=DEV)
    out, idx = bst.decode(q, kc, vc, full, lens, blk, 3)
    torch.cuda.synchronize()
    assert torch.all(idx[1] == -1) and torch.isnan(out[1].float()).all()
    assert not torch.isnan(out[0].float()).any() and not torch.isnan(out[2].float()).any()
