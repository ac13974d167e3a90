"""Comparison rules between the HIP path and the fp64 oracle (test infrastructure).

Index rule: on every row whose k-th and (k+1)-th oracle scores differ by more than 1e-5
relative (denominator max(|s_k|, |s_k+1|)), the selected set must equal the oracle's
bit for bit. On the other rows several answers are right: the GPU set must be a valid
top-k under the oracle's scores, i.e. min over the chosen >= max over the rest minus
1e-5 of the row's magnitude.
Output rule (bf16, fp32): max-abs error <= 2e-2 (bf16) or 1e-4 (fp32), and relative L2
error <= 1e-2 (bf16) or 1e-5 (fp32), computed against the oracle run on the GPU's indices.

Output rule (fp8), derived from the arithmetic (the pages state no fp8 tolerance): the
softmax weights enter the fp8 PV product as e4m3 values. Weights are <= 2^8 and the exact
normaliser is >= 2^7 (the weight of the element that set the row's reference); a normal
e4m3 weight carries relative error <= 2^-4, a subnormal one (< 2^-6) absolute error
<= 2^-10, so |out - ref| <= (2^-4 + n_keys * 2^-17) * max|v| + 2^-8 |ref| (bf16 output
rounding). The max-abs bound doubles the n_keys term for the fp32 sums. Statistically the
errors are far smaller: a weight rounded to e4m3 carries a relative error of rms
2^-4/sqrt(3) ~ 3.6 %, and for outputs that average many keys the relative error of a row is
about that rms whatever the number of keys (the sqrt(sum w^2)/sum w factor of the weights and
the |v|/|out| factor of the average cancel). Rule: relative L2 <= 5e-2 over the tensor and
<= 1e-1 on every query row (the row check catching a single wrong row that the tensor-wide
figures would dilute). Recorded on the GPU (27 fp8 comparisons): 1.6-2.7 % over the tensor,
3.0-4.2 % on the worst row; the CPU simulation of e4m3 weights: 2.2-2.3 %, worst row <= 5.1 %.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle.bsattn_oracle as O

GAP_REL = 1e-5
TOL = {"f32": (1e-4, 1e-5), "bf16": (2e-2, 1e-2), "fp8": (None, 5e-2)}


def dtype_name(t: torch.Tensor) -> str:
    return {torch.float32: "f32", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}[t.dtype]


def to_f64(t: torch.Tensor, descale: float = 1.0) -> np.ndarray:
    """Device/host tensor in storage dtype -> the float64 values the oracle widens."""
    dt = dtype_name(t)
    c = t.detach().cpu().contiguous()
    if dt == "f32":
        return O.widen(c.numpy(), "f32")
    if dt == "bf16":
        return O.widen(c.view(torch.int16).numpy().view(np.uint16), "bf16")
    return O.widen(c.view(torch.uint8).numpy(), "fp8", descale)


def check_idx(gpu_idx: np.ndarray, S: np.ndarray, k: int):
    """gpu_idx [..., k], S [..., nb] oracle scores. Returns a stats dict; asserts the rule."""
    nb = S.shape[-1]
    G = gpu_idx.reshape(-1, k).astype(np.int64)
    Sr = S.reshape(-1, nb)
    assert G.shape[0] == Sr.shape[0]
    assert np.all((G >= 0) & (G < nb)), "index out of range"
    if k > 1:
        assert np.all(np.diff(G, axis=1) > 0), "row not strictly ascending"
    ref = O.select_topk(Sr, k)
    sk, sk1 = O.kth_scores(Sr, k)
    denom = np.maximum(np.abs(sk), np.abs(sk1))
    denom = np.where(np.isfinite(denom), denom, np.abs(sk))
    clear = (sk - sk1) > GAP_REL * denom
    exact_ok = np.all(G == ref, axis=1)
    bad_exact = np.nonzero(clear & ~exact_ok)[0]
    assert bad_exact.size == 0, f"{bad_exact.size} clear rows differ, first {bad_exact[:5]}"
    amb = np.nonzero(~clear)[0]
    mag = np.abs(Sr).max(axis=1)
    for r in amb:
        chosen = np.zeros(nb, dtype=bool)
        chosen[G[r]] = True
        if chosen.all():
            continue
        lo = Sr[r][chosen].min()
        hi = Sr[r][~chosen].max()
        assert lo >= hi - GAP_REL * max(denom[r], mag[r]), f"row {r}: not a valid top-k"
    return {"rows": int(G.shape[0]), "clear": int(clear.sum()), "ambiguous": int(amb.size),
            "ambiguous_differing": int((~exact_ok[amb]).sum()) if amb.size else 0}


def check_random_rows(rows_g: np.ndarray, rows_s: np.ndarray, topk: int, nrand: int, seed: int,
                      rows=None, max_sets: int = 512):
    """Random places [R27] on rows whose top topk - nrand part is not clear under the oracle's
    scores: some split of the GPU row into a top part T and drawn blocks must be right, i.e.
    T (topk - nrand blocks) is a valid top under the index rule's tolerance, and the drawn
    blocks are exactly the oracle's draws given T (the draws depend only on the seed, the row
    number and the blocks outside T). rows_g [R, topk] GPU rows, rows_s [R, nb] oracle scores,
    rows: the row numbers (positions in C order of the whole selection) to check. Returns the
    number of rows checked."""
    import itertools
    nb = rows_s.shape[1]
    kt = topk - nrand
    rows = range(rows_g.shape[0]) if rows is None else rows
    n = 0
    for r in rows:
        g, sc = rows_g[r].astype(np.int64), rows_s[r]
        srt = -np.sort(-sc)
        s_k = srt[kt - 1] if kt > 0 else np.inf
        s_k1 = srt[kt] if kt < nb else -np.inf
        mag = float(np.abs(sc).max())
        tol = GAP_REL * max(abs(s_k) if np.isfinite(s_k) else 0.0,
                            abs(s_k1) if np.isfinite(s_k1) else 0.0, mag)
        sure = [j for j in g if sc[j] > s_k + tol]
        band = [j for j in g if abs(sc[j] - s_k) <= tol]
        need = kt - len(sure)
        assert 0 <= need <= len(band), f"row {r}: no top part of {kt} blocks in the GPU row"
        ok = False
        for m, extra in enumerate(itertools.combinations(band, need)):
            assert m < max_sets, f"row {r}: too many candidate top parts"
            top = np.array(sure + list(extra), dtype=np.int64)
            inside = np.zeros(nb, dtype=bool)
            inside[top] = True
            if kt and (~inside).any() and sc[inside].min() < sc[~inside].max() - tol:
                continue
            tweak = sc.copy()
            tweak[inside] = np.inf                    # the oracle's top part is then exactly T
            want = O.select_topk_random(np.tile(tweak, (r + 1, 1)), topk, nrand, seed)[r]
            if np.array_equal(np.sort(want), np.sort(g)):
                ok = True
                break
        assert ok, f"row {r}: the drawn blocks are not the draws of any valid top part"
        n += 1
    return n


def check_idx_causal(gpu_idx: np.ndarray, S: np.ndarray, k: int):
    """Causal rows [R20]: row i holds min(k, i+1) ascending blocks, the last being i itself,
    then -1; its first min(k, i+1) - 1 entries must pass the index rule above against the
    scores of the blocks j < i. gpu_idx [..., nb, k], S [..., nb, nb] oracle scores."""
    nb = S.shape[-1]
    assert gpu_idx.shape[-2:] == (nb, k)
    for i in range(nb):
        ki = min(k, i + 1)
        rows = gpu_idx[..., i, :]
        assert np.all(rows[..., ki:] == -1), f"row {i}: unused places not -1"
        assert np.all(rows[..., ki - 1] == i), f"row {i}: own block not last"
        if ki > 1:
            check_idx(np.ascontiguousarray(rows[..., :ki - 1]), S[..., i, :i], ki - 1)


GRAD_REL_L2 = 1e-2
GRAD_MAX_REL = 2e-2


def check_grad(gpu: np.ndarray, ref: np.ndarray, name: str = ""):
    """Gradient rule (bf16 backward): relative L2 <= 1e-2 and max-abs <= 2e-2 of max |ref|.
    Derived from the arithmetic: the inputs are the same bf16 values on both sides; the GPU
    rounds P and dS to bf16 (relative error <= 2^-9 each) as MFMA operands and sums in fp32,
    and its rowsum(dO * O) uses the bf16-rounded forward output, so each gradient entry, a sum
    of such products, carries a relative error of a few 2^-9 at most (rms well below 1e-2)."""
    assert not np.isnan(gpu).any(), f"{name}: NaN"
    diff = gpu.astype(np.float64) - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(diff))) / max(float(np.max(np.abs(ref))), 1e-300)
    assert rel <= GRAD_REL_L2 and mx <= GRAD_MAX_REL, (name, rel, mx)
    return rel, mx


def out_errors(gpu_out: np.ndarray, ref: np.ndarray):
    diff = gpu_out.astype(np.float64) - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    rel_l2 = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)) if diff.size else 0.0
    return max_abs, rel_l2


FP8_ROW_REL = 1e-1


def fp8_abs_bound(vmax: float, n_keys: int, ref: np.ndarray) -> float:
    """Worst-case max-abs error of the fp8 path (weights rounded to e4m3, see above)."""
    rmax = float(np.max(np.abs(ref))) if ref.size else 0.0
    return (2.0 ** -4 + n_keys * 2.0 ** -16) * vmax + 2.0 ** -8 * rmax


def fp8_figures(gpu_out: np.ndarray, ref: np.ndarray, vmax: float, n_keys: int) -> dict:
    """What an fp8 comparison achieved next to the rule's bounds: max-abs and its bound,
    relative L2 over the tensor and its bound, the worst query row's relative L2 and its
    bound (printed by the fp8 tests, so that the margin of the rule is on record)."""
    max_abs, rel_l2 = out_errors(gpu_out, ref)
    d = (gpu_out.astype(np.float64) - ref).reshape(-1, ref.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    floor = 1e-3 * float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    row_rel = np.linalg.norm(d, axis=1) / np.maximum(np.linalg.norm(r, axis=1), floor) \
        if r.size else np.zeros(1)
    return {"max_abs": float(f"{max_abs:.3e}"),
            "max_abs_bound": float(f"{fp8_abs_bound(vmax, n_keys, ref):.3e}"),
            "max_abs_over_ref_rms": float(f"{max_abs / max(float(np.sqrt(np.mean(r * r))), 1e-300):.3e}"),
            "rel_l2": float(f"{rel_l2:.3e}"), "rel_l2_bound": TOL["fp8"][1],
            "worst_row_rel_l2": float(f"{float(np.max(row_rel)):.3e}"),
            "worst_row_bound": FP8_ROW_REL}


def check_out(gpu_out: np.ndarray, ref: np.ndarray, dt: str, abs_scale: float = 1.0,
              rel_scale: float = 1.0, fp8_v: tuple | None = None):
    """abs_scale and rel_scale multiply the bounds. The bf16/fp32 bounds above are for
    N(0,1)-like inputs (|out| ~ 0.03, |scores| ~ 10); tests with outputs of O(|v|) or scores
    of O(1e3), whose fp32 dot products alone carry ~1e-4 relative error, pass larger factors.
    fp8: fp8_v = (max |v| over the values read, keys per query row) gives the max-abs bound;
    the last axis of the arrays is the head dimension (one query row per index of the rest)."""
    assert not np.isnan(gpu_out).any(), "output has NaN (unwritten or invalid)"
    max_abs, rel_l2 = out_errors(gpu_out, ref)
    tol_abs, tol_rel = TOL[dt]
    if dt == "fp8":
        assert fp8_v is not None, "fp8 comparisons need (max|v|, keys per row)"
        tol_abs = fp8_abs_bound(fp8_v[0], fp8_v[1], ref)
        if ref.size:
            d = (gpu_out.astype(np.float64) - ref).reshape(-1, ref.shape[-1])
            r = ref.reshape(-1, ref.shape[-1])
            floor = 1e-3 * float(np.sqrt(np.mean(r * r)))
            row_rel = np.linalg.norm(d, axis=1) / np.maximum(np.linalg.norm(r, axis=1), floor)
            worst = int(np.argmax(row_rel))
            assert row_rel[worst] <= FP8_ROW_REL * rel_scale, ("row", worst, float(row_rel[worst]))
    assert max_abs <= tol_abs * abs_scale and rel_l2 <= tol_rel * rel_scale, (max_abs, rel_l2)
    return max_abs, rel_l2
