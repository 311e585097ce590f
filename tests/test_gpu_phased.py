"""GPU parity of batched decode when the routed down product's activations
are too large for one LDS staging but one super-block's columns of them fit
twice: the down kernel then copies super-block after super-block into two
LDS buffers, the next one's copy in flight while the current one computes.
Layer: d_model 256, 64 experts, top-6, expert intermediate 2048 (8
super-blocks), shared intermediate 256, bf16 activations, experts
device-packed (their bytes checked against the oracle's packing) in each
of the three expert formats.  T = 5 selects fewer than 32 distinct experts
on the drawn inputs (the kernel pads the experts it walks to 32, the padding
taking no token); T = 8 and 16 more.  Indices exact, outputs within 2e-3 per
token row."""
import numpy as np
import pytest

from oracle import oracle as O
from bit_quantized_routed_router_amd import ds4moe as D
from bit_quantized_routed_router_amd import synthetic as S
from tests.gpu_helpers import SeededLayer, check_routing, rel_err_rows
from tests.test_gpu_layer import check_used_experts_bytes, oracle_ref

pytestmark = pytest.mark.gpu
TOL = 2e-3
GAP = 1e-4
CFG = S.Config("phased", 256, 64, 6, 2048, 256, 16, "bf16", seed=21)


def stage3_mode(T):
    """The down kernel's staging for T tokens of CFG: 'full', 'phased' or
    'unstaged' (the launcher's byte counts, CB2/Q2K sums included)."""
    Sl = T * CFG.k
    full = Sl * CFG.f * 2 + 2 * Sl * (CFG.f // 16) * 2 + T * CFG.fs * 2
    if full <= 128 * 1024:
        return "full"
    hrows, srows = (Sl + 2) & ~1, (2 * Sl + 32) & ~31  # with the zero rows
    ph = 2 * (hrows * 256 * 2 + srows * 32) + 1024
    return "phased" if ph <= 128 * 1024 and hrows // 2 <= 64 and srows // 32 <= 16 else "unstaged"


@pytest.fixture(scope="module", params=["cb2q2k", "mxfp4", "q4k"])
def layer(request):
    print(f"[setup] phased layer {request.param} (device-packed)", flush=True)
    return SeededLayer(CFG, device_quantize=True, expert_fmt=request.param)


@pytest.mark.parametrize("T", [5, 8, 16])
def test_phased_decode(layer, T):
    assert stage3_mode(T) == "phased"
    x = None
    for v in range(T, T + 64):  # the first input whose fp64 top-k gaps all exceed 1e-4
        cand = layer.x(T=T, variant=v)
        if O.topk_gap(layer.oracle.route(cand, CFG.x_dtype)["logits"], CFG.k).min() > GAP:
            x = cand
            break
    assert x is not None, "no input variant with clear top-k gaps"
    ref = oracle_ref(layer, x)
    nd = len(np.unique(ref["idx"]))
    print(f"phased {layer.expert_fmt} T={T}: {nd} distinct experts", flush=True)
    if T == 5:
        assert nd < 32  # the padded walk
    else:
        assert nd >= 32
    check_used_experts_bytes(layer, ref["idx"])
    got = layer.forward(x, D.MODE_DECODE)
    check_routing(got, ref, CFG.k)
    err = rel_err_rows(got["y"], ref["y"])
    print(f"phased {layer.expert_fmt} T={T} rel err {err:.3e}")
    assert err <= TOL
