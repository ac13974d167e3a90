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


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 value of x >= 0 (the grid decoded by the oracle from all 256 codes)."""
    grid = O.decode_e4m3(np.arange(128, dtype=np.uint8))        # +0 .. 448, ascending
    grid = np.sort(grid[np.isfinite(grid)])
    j = np.clip(np.searchsorted(grid, x), 1, grid.size - 1)
    lo, hi = grid[j - 1], grid[j]
    return np.where(x - lo <= hi - x, lo, hi)


def fp8_weight_output(q, kk, v, idx, blk, scale):
    """Attention with every softmax weight exp2(z - max + 7) rounded to e4m3 and the exact
    normaliser: the arithmetic the fp8 rule bounds."""
    B, N, H, D = q.shape
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            for i in range(N // blk):
                keys = np.concatenate([np.arange(j * blk, (j + 1) * blk) for j in idx[b, h, i]])
                z = q[b, i * blk:(i + 1) * blk, h] @ kk[b, keys, h].T * scale * math.log2(math.e)
                p = np.exp2(z - z.max(axis=1, keepdims=True) + 7)
                out[b, i * blk:(i + 1) * blk, h] = (e4m3_round(p) @ v[b, keys, h]) / p.sum(1)[:, None]
    return out


def test_fp8_rule_accepts_e4m3_weights_and_rejects_one_bad_row():
    q, kk, v, S, idx, out, blk, k, D = setup(3)
    fp8 = fp8_weight_output(q, kk, v, idx, blk, 1 / math.sqrt(D))
    vmax = float(np.abs(v).max())
    max_abs, rel = check_out(fp8, out, "fp8", fp8_v=(vmax, k * blk))
    assert 1e-3 < rel < 5e-2 and max_abs > 0          # the rounding is visible, and within
    # one query row attending to one wrong block: the tensor-wide figures dilute it, the
    # per-row figure does not
    sw = idx.copy()
    sw[0, 1, 3, 0] = next(j for j in range(12) if j not in sw[0, 1, 3])
    bad = O.attend(q, kk, v, sw, blk, 1 / math.sqrt(D), rows=[(0, 1, 3)])
    one_row = fp8.copy()
    one_row[0, 3 * blk + 5, 1] = bad[0, 3 * blk + 5, 1]
    with pytest.raises(AssertionError):
        check_out(one_row, out, "fp8", fp8_v=(vmax, k * blk))
    with pytest.raises(AssertionError):
        check_out(fp8, out, "fp8")                    # fp8 needs its bound's inputs


def test_random_rows_rule():
    """check_random_rows: accepts the oracle's own rows; on a row whose top part is tied at the
    boundary, accepts the other valid split with the draws that split implies and rejects it
    with the draws of the first split; rejects a drawn block that is no draw, and a top part
    without a clearly better block."""
    from tests.parity import check_random_rows
    nb, topk, nrand, seed = 10, 4, 2, 1
    S = np.array([[9.0, 1.0, 8.0, 2.0, 3.0, 0.5, 4.0, 0.1, 0.2, 0.3],
                  [9.0, 7.0, 1.0, 2.0, 3.0, 0.5, 0.1, 0.2, 7.0, 0.3]])   # row 1: tie at top-2
    ref = O.select_topk_random(S, topk, nrand, seed)
    assert check_random_rows(ref, S, topk, nrand, seed) == 2
    assert {0, 1} <= set(ref[1])                 # ties go to the lower index
    tweak = S.copy()
    tweak[1, [0, 8]] = np.inf                    # the other valid top part {0, 8}
    alt = O.select_topk_random(tweak, topk, nrand, seed)[1]
    rows = ref.copy()
    rows[1] = alt
    assert check_random_rows(rows, S, topk, nrand, seed, rows=[1]) == 1
    # top part {0, 8} with the draws of the split {0, 1}
    mixed = np.sort(np.array([0, 8] + [j for j in ref[1] if j not in (0, 1)]))
    assert len(set(mixed)) == topk and not np.array_equal(mixed, np.sort(alt))
    rows[1] = mixed
    with pytest.raises(AssertionError):
        check_random_rows(rows, S, topk, nrand, seed, rows=[1])
    # a drawn block that is not the draw
    drawn = [j for j in ref[0] if j not in (0, 2)]
    spare = next(j for j in range(nb) if j not in ref[0])
    bad = ref.copy()
    bad[0] = np.sort([0, 2, drawn[0], spare])
    with pytest.raises(AssertionError):
        check_random_rows(bad, S, topk, nrand, seed, rows=[0])
    # a top part without the best block (9.0 at block 0)
    worse = ref.copy()
    worse[0] = np.sort([2, 6, 4, 3])
    with pytest.raises(AssertionError):
        check_random_rows(worse, S, topk, nrand, seed, rows=[0])
