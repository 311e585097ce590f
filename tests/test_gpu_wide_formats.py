"""GPU parity of layers whose routed experts are MXFP4 (the model's native
expert format) or Q4K (the Q4 layers of the q2-q4 mix), gate, up and down
alike, against the oracle: the tiny configuration with oracle-packed
experts, and the full DeepSeek V4 Flash shapes with device-packed experts
whose bytes are checked against the oracle's.  Bars as for the CB2/Q2K
layers: indices, counts, offsets and permutation bit-exact, weights within
1e-5, layer outputs within 2e-3 per token row."""
import numpy as np
import pytest

from bit_quantized_routed_router_amd import ds4moe as D
from bit_quantized_routed_router_amd import synthetic as S
from tests.gpu_helpers import SeededLayer, check_routing, rel_err_rows
from tests.test_gpu_layer import check_used_experts_bytes, oracle_ref, slot_tile_kinds

pytestmark = pytest.mark.gpu
TOL = 2e-3


FORMATS = ["mxfp4", "q4k"]


@pytest.fixture(scope="module", params=FORMATS)
def tiny_mx(request):
    print(f"[setup] tiny {request.param} layer (oracle-packed)", flush=True)
    return SeededLayer(S.CONFIGS["tiny"], device_quantize=False, expert_fmt=request.param)


@pytest.mark.parametrize("T", [1, 3, 8, 16, 17, 40])
def test_tiny_mx_decode(tiny_mx, T):
    x = tiny_mx.x(T=T, variant=1100 + T)
    ref = oracle_ref(tiny_mx, x)
    got = tiny_mx.forward(x, D.MODE_DECODE)
    check_routing(got, ref, tiny_mx.cfg.k)
    err = rel_err_rows(got["y"], ref["y"])
    print(f"tiny {tiny_mx.expert_fmt} decode T={T} rel err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("T", [1, 8, 33, 200])
def test_tiny_mx_prefill(tiny_mx, T):
    x = tiny_mx.x(T=T, variant=1200 + T)
    ref = oracle_ref(tiny_mx, x)
    got = tiny_mx.forward(x, D.MODE_PREFILL)
    check_routing(got, ref, tiny_mx.cfg.k)
    err = rel_err_rows(got["y"], ref["y"])
    print(f"tiny {tiny_mx.expert_fmt} prefill T={T} rel err {err:.3e}")
    assert err <= TOL


@pytest.fixture(scope="module", params=FORMATS)
def decode1_mx(request):
    print(f"[setup] decode1 {request.param} layer (device-packed, 256 experts)", flush=True)
    return SeededLayer(S.CONFIGS["decode1"], device_quantize=True, expert_fmt=request.param)


@pytest.mark.parametrize("T", [1, 4])
def test_decode1_mx(decode1_mx, T):
    L = decode1_mx
    for v in range(1300 + 64 * T, 1364 + 64 * T):
        x = L.x(T=T, variant=v)
        from oracle import oracle as O
        if O.topk_gap(L.oracle.route(x, L.cfg.x_dtype)["logits"], L.cfg.k).min() > 1e-4:
            break
    ref = oracle_ref(L, x)
    check_used_experts_bytes(L, ref["idx"])
    got = L.forward(x, D.MODE_DECODE)
    check_routing(got, ref, L.cfg.k)
    err = rel_err_rows(got["y"], ref["y"])
    print(f"decode1 {L.expert_fmt} T={T} rel err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt", FORMATS)
def test_prefill_2048_mx_sampled(fmt):
    """2048-token prefill with the Zipf-shaped loads: routing for every token
    exact, sampled outputs (slots in all three tile kinds) against the
    oracle."""
    print(f"[setup] prefill {fmt} layer (device-packed, Zipf bias)", flush=True)
    L = SeededLayer(S.CONFIGS["prefill"], device_quantize=True, expert_fmt=fmt)
    x = L.x()
    k, T = L.cfg.k, L.cfg.T
    r = L.oracle.route(x, L.cfg.x_dtype)
    kinds = slot_tile_kinds(r["counts"], r["offsets"], r["inv"], r["idx"], k).reshape(T, k)
    g = np.random.default_rng(43)
    sample = [0, T - 1]
    for kind in ("full", "rem", "small"):
        has = np.flatnonzero((kinds == kind).any(axis=1))
        sample += list(g.choice(has, 6, replace=False))
    sample = np.unique(np.array(sample))
    ref = oracle_ref(L, x, tokens=sample)
    got = L.forward(x, D.MODE_PREFILL)
    check_routing(got, ref, k)
    check_used_experts_bytes(L, ref["idx"][sample])
    err = rel_err_rows(got["y"][sample], ref["y"])
    print(f"prefill {fmt} sampled rel err {err:.3e}")
    assert err <= TOL
