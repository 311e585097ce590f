"""GPU parity of batched decode when a group's activations are too large to
stage whole in a block's LDS (T * d_model > 4096 binary16 values): then
each wave of the routed gate/up kernel stages the activations of one
super-block at a time.  d_model 1024, 16 experts, top-2, expert and shared
intermediate 256, fp32 activations (binary16 hi/lo pairs), 8 tokens per
call.  Indices exact, outputs within 2e-3 per token row.  The full-size
bf16 case of the same path is the 16-token decode test of the layer tests."""
import numpy as np
import pytest

from oracle import oracle as O
from bit_quantized_routed_router_amd import ds4moe as D
from bit_quantized_routed_router_amd import synthetic as S
from tests.gpu_helpers import SeededLayer, rel_err_rows

pytestmark = pytest.mark.gpu
TOL = 2e-3
GAP = 1e-4
CFG = S.Config("unstaged8", 1024, 16, 2, 256, 256, 8, "f32", seed=11)


@pytest.fixture(scope="module")
def layer():
    print("[setup] unstaged8 layer (oracle-packed)", flush=True)
    return SeededLayer(CFG, device_quantize=False)


@pytest.mark.parametrize("T", [5, 8, 16])
def test_unstaged_group(layer, T):
    x = None
    for v in range(T, T + 64):  # the first input whose fp64 top-k gaps all exceed 1e-4
        cand = layer.x(T=T, variant=v)
        if O.topk_gap(layer.oracle.route(cand, CFG.x_dtype)["logits"], CFG.k).min() > GAP:
            x = cand
            break
    assert x is not None, "no input variant with clear top-k gaps"
    assert T * CFG.d > 4096  # the unstaged path
    ref = layer.oracle.forward(x, CFG.x_dtype)
    got = layer.forward(x, D.MODE_DECODE)
    assert np.array_equal(got["idx"], ref["idx"])
    err = rel_err_rows(got["y"], ref["y64"])
    print(f"unstaged T={T} rel err {err:.3e}")
    assert err <= TOL
