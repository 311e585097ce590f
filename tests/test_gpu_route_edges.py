"""GPU parity of the routing edge cases against the oracle: exact logit ties,
top-1 routing and expert counts that are not a multiple of the 16-row router
tiles.

Ties are built, not hoped for: the router's rows are repeated in pairs
(row p(2i+1) := row p(2i) for a seeded permutation p), so every logit has an
exact twin on both sides (the oracle's fp64 sum and the GPU's fp32 sum see
the same operands in the same order).  With k odd the k-th and (k+1)-th
largest logits are always such a pair, and the lower expert index must win
(the routing reading: ties go to the lower index).  Input variants are
chosen so that the gap from the tied value to the next lower distinct logit
exceeds TAU for every token, which makes the selected set unique.

Each case runs through the three selection paths of the library: the
one-token finish (T = 1), the batched wave selection of a decode group
(T <= 16) and the per-row top-k of the prefill/route path (T > 16)."""
import numpy as np
import pytest

from bit_quantized_routed_router_amd import ds4moe as D
from bit_quantized_routed_router_amd import synthetic as S
from tests.gpu_helpers import TAU, SeededLayer, check_routing, rel_err_rows

pytestmark = pytest.mark.gpu
TOL = 2e-3

CASES = {
    # name: (config, pair the router rows)
    "e16_k3_ties": (S.Config("e16_k3_ties", 256, 16, 3, 256, 256, 8, "f32", seed=20), True),
    "e16_k1_ties": (S.Config("e16_k1_ties", 256, 16, 1, 256, 256, 8, "f32", seed=21), True),
    "e16_k1": (S.Config("e16_k1", 256, 16, 1, 256, 256, 8, "f32", seed=22), False),
    "e40_k5_ties": (S.Config("e40_k5_ties", 256, 40, 5, 256, 256, 8, "f32", seed=23), True),
    "e40_k6_bf16": (S.Config("e40_k6_bf16", 512, 40, 6, 256, 256, 8, "bf16", seed=24), False),
    "e40_k1": (S.Config("e40_k1", 256, 40, 1, 256, 512, 8, "bf16", seed=25), False),
}


def paired_router(cfg: S.Config) -> np.ndarray:
    r = S.gen_router(cfg).copy()
    p = np.random.default_rng(cfg.seed + 7000).permutation(cfg.E)
    for i in range(0, cfg.E - 1, 2):
        r[p[i + 1]] = r[p[i]]
    return r


def boundary_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token: the k-th largest logit minus the largest logit strictly
    below it (exact ties at the boundary do not count as a gap)."""
    s = -np.sort(-logits, axis=1)
    vk = s[:, k - 1:k]
    below = np.where(s < vk, s, -np.inf).max(axis=1)
    return vk[:, 0] - below


_layers = {}


def layer(name: str) -> SeededLayer:
    if name not in _layers:
        cfg, pair = CASES[name]
        print(f"[setup] {name}: d {cfg.d}, E {cfg.E}, k {cfg.k}, ties {pair}", flush=True)
        _layers[name] = SeededLayer(cfg, device_quantize=False, router=paired_router(cfg) if pair else None)
    return _layers[name]


def clear_input(L: SeededLayer, T: int, v0: int):
    for v in range(v0, v0 + 200):
        x = L.x(T=T, variant=v)
        lg = L.oracle.route(x, L.cfg.x_dtype)["logits"]
        if boundary_gap(lg, L.cfg.k).min() > TAU:
            return x, lg
    raise AssertionError("no input variant with a clear top-k boundary")


def oracle_ref(L: SeededLayer, x):
    r = L.oracle.forward(x, L.cfg.x_dtype)
    return dict(idx=r["idx"], w=r["w"], counts=r["counts"], offsets=r["offsets"], perm=r["perm"], y=r["y64"],
                logits=r["logits"])


def assert_ties_present(L: SeededLayer, logits: np.ndarray):
    """With paired rows and odd k, every token's k-th and (k+1)-th logits tie."""
    cfg, pair = CASES[L.cfg.name]
    if not pair or cfg.k % 2 == 0:
        return
    s = -np.sort(-logits, axis=1)
    assert np.all(s[:, cfg.k - 1] == s[:, cfg.k]), "the constructed tie is missing"


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("T", [1, 7, 40])
def test_route_edges(name, T):
    L = layer(name)
    x, lg = clear_input(L, T, 100 * T)
    assert_ties_present(L, lg)
    ref = oracle_ref(L, x)
    got = L.route(x)
    check_routing(got, ref, L.cfg.k)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("T", [1, 7, 20])
def test_decode_edges(name, T):
    L = layer(name)
    x, lg = clear_input(L, T, 5000 + 100 * T)
    assert_ties_present(L, lg)
    ref = oracle_ref(L, x)
    got = L.forward(x, D.MODE_DECODE)
    check_routing(got, ref, L.cfg.k)
    err = rel_err_rows(got["y"], ref["y"])
    print(f"{name} decode T={T} rel err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("T", [1, 40])
def test_prefill_edges(name, T):
    L = layer(name)
    x, lg = clear_input(L, T, 9000 + 100 * T)
    assert_ties_present(L, lg)
    ref = oracle_ref(L, x)
    got = L.forward(x, D.MODE_PREFILL)
    check_routing(got, ref, L.cfg.k)
    err = rel_err_rows(got["y"], ref["y"])
    print(f"{name} prefill T={T} rel err {err:.3e}")
    assert err <= TOL
