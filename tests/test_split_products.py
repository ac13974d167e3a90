"""The block scores' arithmetic on the bf16 MFMA, simulated on the CPU.

Both score kernels form q.k from three-part bf16 splits of the fp32 pooled values
(x = x0 + x1 + x2, x0 = bf16(x), x1 = bf16(x - x0), x2 = x - x0 - x1) as six products
q0.k0, q0.k1, q1.k0, q0.k2, q1.k1, q2.k0, each exact in fp32. These tests check that:
the split is exact, the three products left out are below 2^-23 of sum_d |q_d k_d|, the sum
in one fp32 accumulator stays at the accuracy of an fp32 matrix product, and a two-part split
would not meet the index rule's 1e-5 (MSA page §3.3: scores as a matrix product; the index
rule is the selection's comparison bar). Rounding is simulated with numpy (RNE to bf16,
float32 sums); no GPU code runs here.
"""
import numpy as np

BOUND_LEFT_OUT = 2.0 ** -23


def bf16_rne(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def split3(x):
    x = np.asarray(x, np.float32)
    x0 = bf16_rne(x)
    r = (x - x0).astype(np.float32)
    x1 = bf16_rne(r)
    x2 = (r - x1).astype(np.float32)
    return x0, x1, x2


def pooled_like(rng, n, D, scale=1 / 8):
    return (rng.standard_normal((n, D)) * scale).astype(np.float32)


def test_split_is_exact_over_the_float_range():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-60, 60, 200_000))).astype(np.float32)
    x0, x1, x2 = split3(x)
    assert np.all(bf16_rne(x2) == x2)                      # the third part is a bf16 value
    assert np.all(x0.astype(np.float64) + x1 + x2 == x.astype(np.float64))


def test_left_out_products_below_bound():
    rng = np.random.default_rng(1)
    for D, scale in ((64, 1 / 8), (128, 1 / 8), (128, 30.0), (64, 1e-3)):
        q, k = pooled_like(rng, 128, D, scale), pooled_like(rng, 96, D, scale)
        Q = [p.astype(np.float64) for p in split3(q)]
        K = [p.astype(np.float64) for p in split3(k)]
        six = (Q[0] @ K[0].T + Q[0] @ K[1].T + Q[1] @ K[0].T + Q[0] @ K[2].T + Q[1] @ K[1].T
               + Q[2] @ K[0].T)
        exact = q.astype(np.float64) @ k.astype(np.float64).T
        mag = np.abs(q.astype(np.float64)) @ np.abs(k.astype(np.float64)).T
        assert np.max(np.abs(six - exact) / mag) <= BOUND_LEFT_OUT


def test_one_accumulator_matches_fp32_matmul_accuracy():
    """The score-matrix kernel adds the six products of each 16-value k-step, smallest first,
    into one fp32 accumulator; simulated with fp32 rounding after every product (the worst
    case), the error stays within a few times an fp32 matrix product's and far inside 1e-5."""
    rng = np.random.default_rng(2)
    D = 128
    q, k = pooled_like(rng, 64, D), pooled_like(rng, 64, D)
    Q, K = split3(q), split3(k)
    acc = np.zeros((64, 64), np.float32)
    for c in range(D // 16):
        for i, j in ((2, 0), (1, 1), (0, 2), (1, 0), (0, 1), (0, 0)):
            for d in range(16 * c, 16 * c + 16):
                acc = (acc + (Q[i][:, d:d + 1] * K[j][None, :, d]).astype(np.float32)).astype(np.float32)
    exact = q.astype(np.float64) @ k.astype(np.float64).T
    mag = np.abs(q.astype(np.float64)) @ np.abs(k.astype(np.float64)).T
    err = np.max(np.abs(acc.astype(np.float64) - exact) / mag)
    f32 = np.max(np.abs((q @ k.T).astype(np.float64) - exact) / mag)
    assert err <= 2e-6 and err <= 8 * max(f32, 2.0 ** -24)


def test_two_part_split_would_not_do():
    """With two parts and three products (q0.k0 + q0.k1 + q1.k0) the left-out terms reach
    2^-16 of sum |q_d k_d|: above the index rule's 1e-5 relative gap for realistic scores."""
    rng = np.random.default_rng(3)
    q, k = pooled_like(rng, 128, 128), pooled_like(rng, 128, 128)
    q0, k0 = bf16_rne(q), bf16_rne(k)
    q1, k1 = bf16_rne((q - q0).astype(np.float32)), bf16_rne((k - k0).astype(np.float32))
    f = lambda a: a.astype(np.float64)
    three = f(q0) @ f(k0).T + f(q0) @ f(k1).T + f(q1) @ f(k0).T
    exact = f(q) @ f(k).T
    rel = np.abs(three - exact) / np.abs(exact)
    assert np.quantile(rel, 0.99) > 1e-5
