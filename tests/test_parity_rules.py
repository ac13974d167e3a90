"""The comparison rules themselves (CPU): they accept the oracle's own answer and reject
a dropped or swapped block, an unsorted row and an out-of-range index."""
import math

import numpy as np
import pytest

import oracle.bsattn_oracle as O
from tests.parity import check_idx, check_out


def setup(seed=0):
    r = np.random.default_rng(seed)
    B, N, H, D, blk, k = 1, 64 * 12, 2, 32, 64, 4
    q, kk, v = (r.standard_normal((B, N, H, D)) for _ in range(3))
    S = O.block_scores(O.pool(q, blk), O.pool(kk, blk))
    idx = O.select_topk(S, k)
    out = O.attend(q, kk, v, idx, blk, 1 / math.sqrt(D))
    return q, kk, v, S, idx, out, blk, k, D


def test_accepts_oracle():
    q, kk, v, S, idx, out, blk, k, D = setup()
    stats = check_idx(idx, S, k)
    assert stats["rows"] == 24
    check_out(out.astype(np.float32), out, "f32")


def test_rejects_swapped_index():
    q, kk, v, S, idx, out, blk, k, D = setup()
    bad = idx.copy()
    row = bad[0, 0, 2]
    row[0] = next(j for j in range(12) if j not in row)
    bad[0, 0, 2] = np.sort(row)
    with pytest.raises(AssertionError):
        check_idx(bad, S, k)


def test_rejects_unsorted_and_out_of_range():
    q, kk, v, S, idx, out, blk, k, D = setup()
    bad = idx.copy()
    bad[0, 1, 0] = bad[0, 1, 0][::-1]
    with pytest.raises(AssertionError):
        check_idx(bad, S, k)
    bad = idx.copy()
    bad[0, 1, 0, -1] = 12
    with pytest.raises(AssertionError):
        check_idx(bad, S, k)


def test_rejects_dropped_or_swapped_block_in_output():
    q, kk, v, S, idx, out, blk, k, D = setup()
    dropped = O.attend(q, kk, v, idx[..., :-1], blk, 1 / math.sqrt(D))
    with pytest.raises(AssertionError):
        check_out(out, dropped, "bf16")
    sw = idx.copy()
    sw[0, 0, 0, 0] = next(j for j in range(12) if j not in sw[0, 0, 0])
    swapped = O.attend(q, kk, v, sw, blk, 1 / math.sqrt(D))
    with pytest.raises(AssertionError):
        check_out(out, swapped, "bf16")


def test_rejects_nan():
    q, kk, v, S, idx, out, blk, k, D = setup()
    o = out.copy()
    o[0, 0, 0, 0] = np.nan
    with pytest.raises(AssertionError):
        check_out(o, out, "bf16")


def test_ambiguous_rows_accept_any_valid_choice():
    S = np.array([[[3.0, 1.0, 2.0, 2.0, 0.0]]])       # k=2: {0,2} or {0,3}
    stats = check_idx(np.array([[[0, 3]]]), S, 2)
    assert stats["ambiguous"] == 1
    with pytest.raises(AssertionError):
        check_idx(np.array([[[0, 1]]]), S, 2)
