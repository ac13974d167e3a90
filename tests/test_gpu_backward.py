"""Parity of the backward (through the C ABI) with the fp64 oracle's gradients, on seeded
inputs; the forward's log-sum-exp output.

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
from tests.parity import check_grad, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def upstream(shape, index):
    """Seeded upstream gradient dO, bf16 (the seed family's sampling stream)."""
    g = torch.Generator(device=DEV).manual_seed(syn.seeds(index)["sample"])
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)


SHAPES = [
    # B, N, Hq, Hkv, D, block, topk
    (2, 64 * 12, 4, 2, 64, 64, 4),      # GQA 2
    (1, 64 * 20, 2, 2, 128, 64, 7),     # D 128
    (1, 64 * 8, 2, 1, 64, 64, 8),       # topk = nb (dense), GQA 2
    (2, 64 * 9, 2, 2, 64, 64, 1),       # topk = 1
    # block 128 (run as 64-token halves over expanded index rows)
    (1, 128 * 10, 4, 2, 128, 128, 4),   # GQA 2, D 128
    (2, 128 * 6, 2, 2, 64, 128, 3),     # D 64
    (1, 128 * 5, 2, 1, 64, 128, 5),     # topk = nb (dense), GQA 2
    (1, 128 * 7, 2, 2, 128, 128, 1),    # topk = 1: causal rows hold only the own block
]


def run_case(shape, causal, index=31):
    B, N, Hq, Hkv, D, blk, topk = shape
    q, k, v, _ = syn.iid_inputs(B, N, Hq, Hkv, D, "bf16", index=index, device=DEV)
    idx = bst.select(q, k, blk, topk, causal=causal)
    out, lse = bst.forward(q, k, v, idx, causal=causal, return_lse=True)
    dout = upstream(out.shape, index)
    dq, dk, dv = bst.backward(q, k, v, idx, out, dout, lse, causal=causal)
    torch.cuda.synchronize()
    return q, k, v, idx, out, lse, dout, (dq, dk, dv)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_backward(shape, causal):
    B, N, Hq, Hkv, D, blk, topk = shape
    say(f"[backward] causal={causal} shape={shape}")
    q, k, v, idx, out, lse, dout, grads = run_case(shape, causal)
    qo, ko, vo, go = (to_f64(x) for x in (q, k, v, dout))
    gidx = idx.cpu().numpy()
    scale = 1 / math.sqrt(D)
    ref_lse = O.attend_lse(qo, ko, gidx, blk, scale, causal=causal)
    # the bf16 forward sums its normaliser from the bf16-rounded weights (relative error
    # <= 2^-9 each), the one its output is divided by: |log l~ - log l| <= 2^-9, plus fp32
    # rounding of the scores
    err = np.max(np.abs(lse.cpu().numpy() - ref_lse))
    assert err <= 2.0 ** -9 + 1e-5 * max(1.0, np.abs(ref_lse).max()), err
    refs = O.attend_backward(qo, ko, vo, gidx, blk, scale, go, causal=causal)
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        say(f"   {name}: rel_l2, max_rel =", check_grad(g.cpu().numpy(), r, name))
    # negative control: the gradients of a selection with one block dropped differ
    if topk > 2 and not causal:
        fewer = O.attend_backward(qo, ko, vo, gidx[..., :-1], blk, scale, go)
        with pytest.raises(AssertionError):
            check_grad(grads[0].cpu().numpy(), fewer[0], "dq")


def test_backward_deterministic():
    say("[backward determinism]")
    shape = (2, 64 * 12, 4, 1, 64, 64, 5)
    a = run_case(shape, False, index=32)
    b = run_case(shape, False, index=32)
    for x, y in zip(a[-1], b[-1]):
        assert torch.equal(x, y)


@pytest.mark.slow
def test_backward_sparseformer_sampled_heads():
    """The page's benchmark shape: the gradients of 3 sampled (batch, head) pairs (all of
    their query and key blocks) against the oracle."""
    w = syn.WORKLOADS["sparseformer_n8192_bf16"]
    say("[backward full size]", w)
    q, k, v, ds, _ = syn.workload_inputs(w, device=DEV)
    topk = O.topk_count(w.ratio, w.nb)
    idx = bst.select(q, k, w.block, topk)
    out, lse = bst.forward(q, k, v, idx, return_lse=True)
    dout = upstream(out.shape, w.index)
    dq, dk, dv = bst.backward(q, k, v, idx, out, dout, lse)
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    rows = syn.sample_rows(3, w.B * w.Hq, w.index)
    for r in rows:
        b, h = r // w.Hq, r % w.Hq
        say(f"  (b, h) = ({b}, {h})")
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        qo, ko, vo, go = (to_f64(x[sl].contiguous()) for x in (q, k, v, dout))
        refs = O.attend_backward(qo, ko, vo, gidx[b:b + 1, h:h + 1], w.block,
                                 1 / math.sqrt(w.D), go)
        for name, g, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
            check_grad(g[sl].cpu().numpy(), ref, name)
