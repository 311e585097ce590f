"""Pins for the oracle's router, top-k, gate weights and token grouping (CPU)."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import oracle as O
from bit_quantized_routed_router_amd import synthetic as S


def test_router_logits_match_library_matmul():
    cfg = S.CONFIGS["tiny"]
    x = S.gen_x(cfg)
    wr = S.gen_router(cfg)
    bias = np.linspace(-1, 1, cfg.E).astype(np.float32)
    X = O.x_to_f64(x, cfg.x_dtype)
    got = O.router_logits(X, wr, bias)
    ref = X @ wr.view(np.float16).astype(np.float64).T + bias.astype(np.float64)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_x_conversion_exact():
    x = np.array([[1.5, -2.0, 3.0e-20]], dtype=np.float32)
    assert np.array_equal(O.x_to_f64(x, "f32"), x.astype(np.float64))
    b = S.f32_to_bf16_bits(x)
    assert np.array_equal(O.x_to_f64(b, "bf16"), S.bf16_bits_to_f32(b).astype(np.float64))


@pytest.mark.parametrize("T,E,k", [(1, 16, 2), (33, 256, 6), (5, 7, 7), (9, 64, 1)])
def test_topk_equals_full_sort(T, E, k):
    g = np.random.default_rng(T * 1000 + E)
    logits = g.standard_normal((T, E))
    idx, w = O.topk(logits, k)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))  # by logit desc, then index asc
        ref = np.sort(order[:k])
        assert np.array_equal(idx[t], ref)
        assert np.allclose(w[t], softmax(logits[t, ref]), rtol=1e-13, atol=0)
        assert abs(w[t].sum() - 1.0) < 1e-12


def test_topk_ties_go_to_lower_index():
    logits = np.array([[0.5, 2.0, 2.0, 1.0, 2.0, 0.1]])
    idx, w = O.topk(logits, 2)
    assert list(idx[0]) == [1, 2]
    assert np.allclose(w[0], [0.5, 0.5])
    idx, _ = O.topk(logits, 4)
    assert list(idx[0]) == [1, 2, 3, 4]


def test_topk_k_equals_one_weight_is_exactly_one():
    logits = np.random.default_rng(3).standard_normal((10, 12))
    idx, w = O.topk(logits, 1)
    assert np.array_equal(idx[:, 0], np.argmax(logits, axis=1))
    assert (w == 1.0).all()


@pytest.mark.parametrize("T,E,k", [(8, 16, 2), (16, 256, 6), (1, 256, 6), (50, 8, 3)])
def test_permute_brute_force(T, E, k):
    g = np.random.default_rng(T + E + k)
    idx = np.stack([np.sort(g.permutation(E)[:k]) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = O.permute(idx, E)
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k and (np.diff(offsets) >= 0).all()
    ref = sorted(range(T * k), key=lambda s: (idx[s // k, s % k], s // k))
    assert list(perm) == ref
    assert np.array_equal(np.sort(perm), np.arange(T * k))
    assert np.array_equal(inv[perm], np.arange(T * k))
    for e in range(E):
        seg = perm[offsets[e]: offsets[e + 1]]
        assert all(idx[s // k, s % k] == e for s in seg)


def test_topk_gap_helper():
    logits = np.array([[3.0, 1.0, 2.0, 2.5]])
    assert np.allclose(O.topk_gap(logits, 2), [0.5])


def test_configs_carry_the_selected_seeds():
    """synthetic.CONFIGS holds the variants find_seeds.py selected."""
    import json
    import os
    sel = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "seeds.json")))
    for name in ("decode1", "decode16", "prefill"):
        c = S.CONFIGS[name]
        assert c.router_variant == sel[name]["router_variant"]
        assert c.x_variant == sel[name]["x_variant"]
    assert S.CONFIGS["prefill"].zipf_beta == sel["prefill"]["zipf_beta"]


@pytest.mark.slow
def test_decode1_gap_rule_holds():
    cfg = S.CONFIGS["decode1"]
    X = O.x_to_f64(S.gen_x(cfg), cfg.x_dtype)
    L = O.router_logits(X, S.gen_router(cfg), S.gen_bias(cfg))
    assert O.topk_gap(L, cfg.k).min() > 1e-4
