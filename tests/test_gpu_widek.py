"""GPU parity at a shape wider than the prefill kernels' staged scale range.

d_model 4352 gives 17 CB2 blocks per gate/up row, one more than the 16 whose
scales a gate/up block stages in LDS.  Expert intermediate 2304 gives 9 Q2K
blocks per down row, one more than the 8 staged by the small-tile down
kernel.  The last block of every row therefore takes its scales from memory
inside the same chunk loop.  The layer has 16 experts, top-2 and shared
intermediate 256.  300 tokens spread about 37 slots over each expert, so
both the small-tile list (at most 32 slots) and the large one are used.

Routing is compared bit for bit for every token.  Outputs of a seeded
sample of tokens are compared with the oracle within 2e-3 per row, for
bf16 and fp32 activations.  The input variant is the first whose fp64 gap
between the 2nd and 3rd logit exceeds 1e-4 for every token, so that the
expert sets are unique against the GPU's fp32 accumulation."""
import numpy as np
import pytest

from oracle import oracle as O
from bit_quantized_routed_router_amd import ds4moe as D
from bit_quantized_routed_router_amd import synthetic as S
from tests.gpu_helpers import SeededLayer, check_routing, rel_err_rows

pytestmark = pytest.mark.gpu
TOL = 2e-3
GAP = 1e-4


def clear_input(L: SeededLayer):
    for v in range(64):
        x = L.x(variant=v)
        logits = L.oracle.route(x, L.cfg.x_dtype)["logits"]
        if O.topk_gap(logits, L.cfg.k).min() > GAP:
            return x
    raise AssertionError("no input variant with a clear top-k gap")


@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_prefill_past_staged_scales(xdt):
    cfg = S.Config("widek", 4352, 16, 2, 2304, 256, 300, xdt, seed=21)
    print(f"[setup] widek layer ({xdt}, device-packed)", flush=True)
    L = SeededLayer(cfg, device_quantize=True)
    x = clear_input(L)
    sample = np.sort(np.random.default_rng(7).choice(cfg.T, 20, replace=False))
    sample = np.unique(np.concatenate([sample, [0, cfg.T - 1]]))
    r = L.oracle.forward(x, cfg.x_dtype, tokens=sample)
    ref = dict(idx=r["idx"], w=r["w"], counts=r["counts"], offsets=r["offsets"], perm=r["perm"])
    got = L.forward(x, D.MODE_PREFILL)
    check_routing(got, ref, cfg.k)
    counts = np.asarray(r["counts"])
    assert (counts <= 32).any() and (counts > 32).any(), "both tile lists must be used"
    for e in np.unique(r["idx"][sample]):
        for g, o in zip(L.device_expert_bytes(int(e)), L.oracle_expert(int(e))):
            assert np.array_equal(g, o), f"device packing of expert {e} differs from the oracle's"
    err = rel_err_rows(got["y"][sample], r["y64"])
    print(f"widek {xdt} prefill sampled rel err {err:.3e}", flush=True)
    assert err <= TOL
