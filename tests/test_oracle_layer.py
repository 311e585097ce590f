"""Pins for the oracle's expert math and full layer (CPU)."""
import numpy as np
import pytest
from scipy.special import expit

from oracle import oracle as O
from bit_quantized_routed_router_amd import synthetic as S


def tiny_layer(cfg=None, k=None, bias=None):
    cfg = cfg or S.CONFIGS["tiny"]
    k = cfg.k if k is None else k
    wr = S.gen_router(cfg)
    sg, su, sd = S.gen_shared(cfg)
    packs = {}
    for e in range(cfg.E):
        g, u, dn = S.gen_expert(cfg, e)
        packs[e] = (O.cb2_quantize(g), O.cb2_quantize(u), O.q2k_quantize(dn))
    return O.Layer(cfg.d, cfg.E, k, cfg.f, cfg.fs, wr, bias, sg, su, sd, packs)


def test_swiglu_matches_scipy():
    g = np.linspace(-30, 30, 101)
    u = np.cos(g)
    assert np.allclose(O.swiglu(g, u), g * expit(g) * u, rtol=1e-14, atol=1e-300)


def test_f16_matmul_matches_numpy():
    rng = np.random.default_rng(0)
    w = S.f32_to_f16_bits(rng.standard_normal((40, 256)).astype(np.float32) * 0.02)
    X = rng.standard_normal((3, 256))
    ref = X @ w.view(np.float16).astype(np.float64).T
    assert np.allclose(O.f16_matmul(w, X), ref, rtol=1e-13, atol=1e-15)


def test_packed_matmuls_match_numpy_on_dequantized():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((48, 512)) * 0.02).astype(np.float32)
    X = rng.standard_normal((5, 512))
    p = O.cb2_quantize(w)
    ref = X @ O.cb2_dequantize(p, 48, 512).astype(np.float64).T
    assert np.allclose(O.cb2_matmul(p, 48, 512, X), ref, rtol=1e-12, atol=1e-14)
    q = O.q2k_quantize(w)
    ref = X @ O.q2k_dequantize(q, 48, 512).astype(np.float64).T
    assert np.allclose(O.q2k_matmul(q, 48, 512, X), ref, rtol=1e-12, atol=1e-14)


def test_expert_equals_numpy_swiglu_chain():
    cfg = S.CONFIGS["tiny"]
    L = tiny_layer()
    X = O.x_to_f64(S.gen_x(cfg), "f32")
    e = 3
    gp, up, dp = L.expert(e)
    G = O.cb2_dequantize(gp, cfg.f, cfg.d).astype(np.float64)
    U = O.cb2_dequantize(up, cfg.f, cfg.d).astype(np.float64)
    D = O.q2k_dequantize(dp, cfg.d, cfg.f).astype(np.float64)
    gx, ux = X @ G.T, X @ U.T
    ref = (gx * expit(gx) * ux) @ D.T
    got = L.expert_out(e, X)
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_layer_equals_dense_all_experts():
    """Computing every expert for every token and combining with a dense,
    zero-padded weight matrix gives the routed result."""
    cfg = S.CONFIGS["tiny"]
    L = tiny_layer()
    x = S.gen_x(cfg)
    r = L.forward(x, "f32")
    X = r["X"]
    allout = np.stack([L.expert_out(e, X) for e in range(cfg.E)], axis=1)  # [T, E, d]
    W = np.zeros((cfg.T, cfg.E))
    for t in range(cfg.T):
        W[t, r["idx"][t]] = r["w"][t]
    sg = X @ L.sh_gate.view(np.float16).astype(np.float64).T
    su = X @ L.sh_up.view(np.float16).astype(np.float64).T
    ys = (sg * expit(sg) * su) @ L.sh_down.view(np.float16).astype(np.float64).T
    ref = ys + np.einsum("te,ted->td", W, allout)
    rel = np.abs(r["y64"] - ref).max() / np.abs(ref).max()
    assert rel < 1e-12
    assert np.array_equal(r["y"], r["y64"].astype(np.float32))


def test_layer_k1_is_shared_plus_one_expert():
    cfg = S.CONFIGS["tiny"]
    L = tiny_layer(k=1)
    x = S.gen_x(cfg)
    r = L.forward(x, "f32")
    X = r["X"]
    for t in range(cfg.T):
        e = int(r["idx"][t, 0])
        ref = L.shared(X[t:t + 1])[0] + L.expert_out(e, X[t:t + 1])[0]
        assert np.allclose(r["y64"][t], ref, rtol=1e-13, atol=1e-13)


def test_layer_token_subset_matches_full():
    cfg = S.CONFIGS["tiny"]
    L = tiny_layer()
    x = S.gen_x(cfg)
    full = L.forward(x, "f32")
    sub = L.forward(x, "f32", tokens=[6, 1])
    assert np.array_equal(sub["y64"], full["y64"][[6, 1]])
    assert np.array_equal(sub["perm"], full["perm"])


def test_tiny_config_gap_rule_holds():
    """The tiny workload's router keeps every top-k gap above 1e-4."""
    cfg = S.CONFIGS["tiny"]
    X = O.x_to_f64(S.gen_x(cfg), "f32")
    logits = O.router_logits(X, S.gen_router(cfg), None)
    assert O.topk_gap(logits, cfg.k).min() > 1e-4


def test_mxfp4_matmul_and_expert_chain_match_numpy():
    """MXFP4 experts: the oracle's product and the layer's expert chain equal
    numpy fp64 on the dequantized matrices."""
    cfg = S.CONFIGS["tiny"]
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((48, 512)) * 0.02).astype(np.float32)
    X = rng.standard_normal((5, 512))
    p = O.mx4_quantize(w)
    ref = X @ O.mx4_dequantize(p, 48, 512).astype(np.float64).T
    assert np.allclose(O.mx4_matmul(p, 48, 512, X), ref, rtol=1e-12, atol=1e-14)
    packs = {}
    for e in range(cfg.E):
        g, u, dn = S.gen_expert(cfg, e)
        packs[e] = (O.mx4_quantize(g), O.mx4_quantize(u), O.mx4_quantize(dn))
    sg, su, sd = S.gen_shared(cfg)
    L = O.Layer(cfg.d, cfg.E, cfg.k, cfg.f, cfg.fs, S.gen_router(cfg), None, sg, su, sd, packs, expert_fmt="mxfp4")
    Xt = O.x_to_f64(S.gen_x(cfg), "f32")
    G = O.mx4_dequantize(packs[5][0], cfg.f, cfg.d).astype(np.float64)
    U = O.mx4_dequantize(packs[5][1], cfg.f, cfg.d).astype(np.float64)
    D = O.mx4_dequantize(packs[5][2], cfg.d, cfg.f).astype(np.float64)
    gx, ux = Xt @ G.T, Xt @ U.T
    assert np.allclose(L.expert_out(5, Xt), (gx * expit(gx) * ux) @ D.T, rtol=1e-11, atol=1e-12)


def test_q4k_matmul_and_expert_chain_match_numpy():
    """Q4K experts: the oracle's product and the layer's expert chain equal
    numpy fp64 on the dequantized matrices."""
    cfg = S.CONFIGS["tiny"]
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((48, 512)) * 0.02).astype(np.float32)
    X = rng.standard_normal((5, 512))
    p = O.q4k_quantize(w)
    ref = X @ O.q4k_dequantize(p, 48, 512).astype(np.float64).T
    assert np.allclose(O.q4k_matmul(p, 48, 512, X), ref, rtol=1e-12, atol=1e-14)
    packs = {}
    for e in range(cfg.E):
        g, u, dn = S.gen_expert(cfg, e)
        packs[e] = (O.q4k_quantize(g), O.q4k_quantize(u), O.q4k_quantize(dn))
    sg, su, sd = S.gen_shared(cfg)
    L = O.Layer(cfg.d, cfg.E, cfg.k, cfg.f, cfg.fs, S.gen_router(cfg), None, sg, su, sd, packs, expert_fmt="q4k")
    Xt = O.x_to_f64(S.gen_x(cfg), "f32")
    G = O.q4k_dequantize(packs[9][0], cfg.f, cfg.d).astype(np.float64)
    U = O.q4k_dequantize(packs[9][1], cfg.f, cfg.d).astype(np.float64)
    D = O.q4k_dequantize(packs[9][2], cfg.d, cfg.f).astype(np.float64)
    gx, ux = Xt @ G.T, Xt @ U.T
    assert np.allclose(L.expert_out(9, Xt), (gx * expit(gx) * ux) @ D.T, rtol=1e-11, atol=1e-12)
