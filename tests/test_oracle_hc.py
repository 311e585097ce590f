"""Pins for the oracle's hyper-connection mixer (CPU only): Sinkhorn values
worked by hand (tests/golden/hc_sinkhorn.json), closed forms of the Sinkhorn
limit (rank-one, equal-row-sum circulant and 2x2 blocks, whose doubly
stochastic limit is fixed by the cross ratio), the projection's flattening,
grouping and RMS normalisation through one-hot projections, and the expand
step's conservation law, which holds exactly because the last half-step
normalises columns."""
import json
import math
import os

import numpy as np

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sig(v):
    return 1.0 / (1.0 + math.exp(-v))


def test_sinkhorn_hand_worked_iterations():
    fx = json.load(open(os.path.join(GOLDEN, "hc_sinkhorn.json")))
    Z = np.log(np.array(fx["exp_Z"], dtype=np.float64))
    for it, v in fx["iterations"].items():
        want = np.array(v["num"], dtype=np.float64) / np.array(v["den"], dtype=np.float64)
        assert np.allclose(O.sinkhorn(Z, int(it)), want, rtol=1e-14, atol=0), it


def test_sinkhorn_rank_one_is_uniform():
    a = np.array([0.3, -1.2, 2.0, 0.7])
    b = np.array([-0.5, 1.5, 0.1, -2.2])
    M = O.sinkhorn(a[:, None] + b[None, :], 20)
    assert np.allclose(M, 0.25, rtol=0, atol=1e-15)


def test_sinkhorn_circulant_closed_form():
    """Equal row and column sums: exp(Z) / row sum after the first
    half-step, unchanged after."""
    c = np.array([3.0, -0.5, 0.25, 1.0])
    Z = np.array([[c[(j - i) % 4] for j in range(4)] for i in range(4)])
    want = np.exp(Z) / np.exp(c).sum()
    for it in (1, 20):
        assert np.allclose(O.sinkhorn(Z, it), want, rtol=1e-14, atol=0)


def test_sinkhorn_two_by_two_blocks_cross_ratio():
    """Blocks [[a, b], [c, d]] (zeros elsewhere) tend to [[p, 1-p], [1-p, p]]
    with p / (1 - p) = sqrt(ad / bc); these blocks converge well inside 20
    iterations."""
    blocks = [np.exp([[0.3, -0.4], [0.9, 0.1]]), np.array([[2.0, 1.0], [1.0, 3.0]])]
    Z = np.full((4, 4), -800.0)  # exp underflows to exactly 0
    Z[:2, :2] = np.log(blocks[0])
    Z[2:, 2:] = np.log(blocks[1])
    M = O.sinkhorn(Z, 20)
    for bi, B in enumerate(blocks):
        (a, b), (c, d) = B
        p = math.sqrt(a * d) / (math.sqrt(a * d) + math.sqrt(b * c))
        s = slice(2 * bi, 2 * bi + 2)
        assert np.allclose(M[s, s], [[p, 1 - p], [1 - p, p]], rtol=0, atol=1e-13)
    assert not M[:2, 2:].any() and not M[2:, :2].any()


def slow_mixer():
    """A 4x4 logit matrix whose rows are still far from summing to one after
    20 iterations (columns do, exactly)."""
    return np.array([[3.904, 0.435, -0.756, 2.397], [5.513, -4.563, 5.61, -5.888],
                     [-7.276, -5.813, 7.876, -4.945], [-1.467, 5.864, -2.746, 5.925]])


def test_sinkhorn_columns_exact_rows_not_yet():
    M = O.sinkhorn(slow_mixer(), 20)
    assert np.allclose(M.sum(0), 1.0, rtol=0, atol=1e-15)
    assert np.abs(M.sum(1) - 1.0).max() > 1e-3
    # a row shift of the logits is removed exactly by the first row step
    M2 = O.sinkhorn(slow_mixer() + np.array([1.5, -2.0, 0.25, 3.0])[:, None], 20)
    assert np.allclose(M2, M, rtol=1e-12, atol=0)


def _pre(X, phi, bias, alpha=(1.0, 1.0, 1.0), eps=1e-6, iters=20):
    return O.hc_pre(X[None], phi, bias, alpha, eps, iters)


def test_hc_pre_zero_projection_is_bias_only():
    rng = np.random.default_rng(1)
    n, d = 4, 64
    X = rng.standard_normal((n, d))
    bias = rng.standard_normal(24)
    c = np.array([2.0, 0.0, -1.0, 0.5])
    bias[8:] = [c[(j - i) % 4] for i in range(4) for j in range(4)]
    coef, xin = _pre(X, np.zeros((24, n * d)), bias)
    coef, xin = coef[0], xin[0]
    for i in range(4):
        assert coef[i] == sig(bias[i])
        assert abs(coef[4 + i] - 2 * sig(bias[4 + i])) <= 4e-16
    M = coef[8:].reshape(4, 4)
    assert np.allclose(M, np.exp(bias[8:].reshape(4, 4)) / np.exp(c).sum(), rtol=1e-14, atol=0)
    want = sum(coef[i] * X[i] for i in range(4))
    assert np.allclose(xin, want, rtol=1e-15, atol=1e-15)


def test_hc_pre_one_hot_projection_pins_indexing_groups_and_rms():
    """Row o of phi one-hot at flat index k_o = i*d + c: z_o = alpha_g *
    X[i][c] / rms(X) + bias_o, with rms over all n*d values plus eps."""
    rng = np.random.default_rng(2)
    n, d, eps = 4, 64, 1e-3
    X = rng.standard_normal((n, d)) * np.array([0.5, 1.0, 2.0, 4.0])[:, None]
    rms = math.sqrt(float(np.mean(X.astype(np.float64) ** 2)) + eps)
    alpha = (0.5, 2.0, 3.0)
    phi = np.zeros((24, n * d))
    picks = [(i % 4, (7 * i + 3) % d) for i in range(8)]
    for o, (i, c) in enumerate(picks):
        phi[o, i * d + c] = 1.0
    # residual rows: circulant pattern Z[i][j] = v[(j - i) % 4] from four picked entries
    circ = [(0, 5), (1, 9), (2, 33), (3, 60)]
    for i in range(4):
        for j in range(4):
            si, sc = circ[(j - i) % 4]
            phi[8 + 4 * i + j, si * d + sc] = 1.0
    bias = np.zeros(24)
    bias[:8] = np.linspace(-0.5, 0.5, 8)
    coef, _ = _pre(X, phi, bias, alpha, eps)
    coef = coef[0]
    for o, (i, c) in enumerate(picks):
        z = (alpha[0] if o < 4 else alpha[1]) * X[i, c] / rms + bias[o]
        want = sig(z) if o < 4 else 2 * sig(z)
        assert abs(coef[o] - want) <= 1e-14, o
    v = np.array([alpha[2] * X[si, sc] / rms for si, sc in circ])
    Zc = np.array([[v[(j - i) % 4] for j in range(4)] for i in range(4)])
    assert np.allclose(coef[8:].reshape(4, 4), np.exp(Zc) / np.exp(v).sum(), rtol=1e-13, atol=0)


def test_hc_pre_scale_invariant_without_eps():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((4, 64))
    phi = rng.standard_normal((24, 256)) / 16
    bias = rng.standard_normal(24)
    c1, x1 = _pre(X, phi, bias, eps=0.0)
    c2, x2 = _pre(8.0 * X, phi, bias, eps=0.0)
    assert np.allclose(c1, c2, rtol=1e-13, atol=1e-15)
    assert np.allclose(8.0 * x1, x2, rtol=1e-13, atol=1e-13)


def test_hc_post_uniform_mixer_is_mean_plus_post():
    rng = np.random.default_rng(4)
    T, n, d = 3, 4, 64
    X = rng.standard_normal((T, n, d))
    y = rng.standard_normal((T, d))
    coef = np.zeros((T, 24))
    coef[:, 4:8] = rng.uniform(0, 2, (T, 4))
    coef[:, 8:] = 0.25
    out = O.hc_post(X, y, coef)
    want = X.mean(axis=1, keepdims=True) + coef[:, 4:8, None] * y[:, None, :]
    assert np.allclose(out, want, rtol=1e-14, atol=1e-14)


def test_hc_post_conserves_stream_sum():
    """Columns of M sum to one, so sum_i X'_i = sum_j X_j + (sum_i post_i) y,
    while the rows of this mixer do not: a transposed M fails."""
    rng = np.random.default_rng(5)
    T, n, d = 2, 4, 128
    X = rng.standard_normal((T, n, d))
    y = rng.standard_normal((T, d))
    coef = np.zeros((T, 24))
    coef[:, 4:8] = rng.uniform(0, 2, (T, 4))
    coef[:, 8:] = O.sinkhorn(slow_mixer(), 20).ravel()
    out = O.hc_post(X, y, coef)
    want = X.sum(axis=1) + coef[:, 4:8].sum(axis=1)[:, None] * y
    assert np.allclose(out.sum(axis=1), want, rtol=0, atol=1e-12)
    bad = O.hc_post(X, y, np.concatenate([coef[:, :8], coef[:, 8:].reshape(T, 4, 4).transpose(0, 2, 1)
                                          .reshape(T, 16)], axis=1))
    assert not np.allclose(bad.sum(axis=1), want, rtol=0, atol=1e-6)


def test_hc_post_identity_limit():
    """A strongly diagonal circulant mixer is the closed form
    exp(Z) / row sum; with it X' = M X + post y row by row."""
    rng = np.random.default_rng(6)
    X = rng.standard_normal((1, 4, 32))
    y = rng.standard_normal((1, 32))
    c = np.array([30.0, 0.0, 0.0, 0.0])
    Z = np.array([[c[(j - i) % 4] for j in range(4)] for i in range(4)])
    M = O.sinkhorn(Z, 20)
    diag = math.exp(30.0) / (math.exp(30.0) + 3.0)
    assert np.allclose(np.diag(M), diag, rtol=1e-15, atol=0)
    coef = np.concatenate([np.zeros(4), np.ones(4), M.ravel()])[None]
    out = O.hc_post(X, y, coef)
    assert np.allclose(out[0], M @ X[0] + y[0][None, :], rtol=1e-14, atol=1e-14)


def test_hc_thread_independence():
    from bit_quantized_routed_router_amd import synthetic as S
    X, phi, bias, alpha, y = S.gen_hc(256, 6)
    n0 = O.max_threads()
    try:
        O.set_threads(1)
        c1, x1 = O.hc_pre(X, phi, bias, alpha, S.HC_EPS, S.HC_SINKHORN_ITERS)
        O.set_threads(4)
        c4, x4 = O.hc_pre(X, phi, bias, alpha, S.HC_EPS, S.HC_SINKHORN_ITERS)
    finally:
        O.set_threads(n0)
    assert np.array_equal(c1, c4) and np.array_equal(x1, x4)
