"""The workspace-free decode entry point (ds4moe_forward_decode_static)
against ds4moe_forward_decode with a caller workspace: the same kernels run,
so outputs, expert indices and gate weights must be equal bit for bit.  Two
calls in a row on the library's one device array, the second with a smaller
input, so that the second call sees whatever the first one left there."""
import numpy as np
import pytest
import torch

from bit_quantized_routed_router_amd import ds4moe as D
from bit_quantized_routed_router_amd import synthetic as S
from tests.gpu_helpers import SeededLayer, dev, host, rel_err_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    print("[setup] tiny layer (oracle-packed)", flush=True)
    return SeededLayer(S.CONFIGS["tiny"], device_quantize=False)


def run_both(L: SeededLayer, x: np.ndarray):
    T, c = x.shape[0], L.cfg
    xd = dev(x)
    outs = []
    for static in (True, False):
        y = torch.full((T, c.d), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((T, c.k), -1, dtype=torch.int32, device="cuda")
        w = torch.full((T, c.k), float("nan"), dtype=torch.float32, device="cuda")
        if static:
            D.forward_decode_static(L.layer.desc, xd, L.x_dtype(), T, y, idx, w)
        else:
            ws, n = L.layer.workspace(T, D.MODE_DECODE)
            D.forward_decode(L.layer.desc, xd, L.x_dtype(), T, y, idx, w, ws, n)
        torch.cuda.synchronize()
        outs.append((host(y), host(idx), host(w)))
    return outs


@pytest.mark.parametrize("Ts", [(16, 3), (40, 1)])
def test_static_decode_equals_workspace_decode(tiny, Ts):
    for n, T in enumerate(Ts):
        x = tiny.x(T=T, variant=600 + 10 * T + n)
        (ys, is_, ws_), (yw, iw, ww) = run_both(tiny, x)
        assert np.array_equal(is_, iw)
        assert np.array_equal(ws_, ww)
        assert np.array_equal(ys, yw), f"call {n} (T={T}): static and workspace outputs differ"
        ref = tiny.oracle.forward(x, tiny.cfg.x_dtype)
        assert np.array_equal(is_, ref["idx"])
        assert rel_err_rows(ys, ref["y64"]) <= 2e-3


def test_static_decode_full_shape_one_token():
    """decode1 shape (d 4096, E 256, top-6, f 2048): one token, then the same
    layer at T = 1 again after a 4-token call."""
    L = SeededLayer(S.CONFIGS["decode1"], device_quantize=True)
    for n, T in enumerate((4, 1)):
        x = L.x(T=T, variant=700 + n)
        (ys, is_, ws_), (yw, iw, ww) = run_both(L, x)
        assert np.array_equal(is_, iw) and np.array_equal(ws_, ww)
        assert np.array_equal(ys, yw), f"call {n} (T={T}): static and workspace outputs differ"
