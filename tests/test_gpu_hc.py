"""GPU parity of the hyper-connection mixer (ds4moe_hc_pre / ds4moe_hc_post)
against the oracle, on seeded streams with the note's shape (4 streams of
4096, 20 Sinkhorn iterations) and on a small width that exercises both K-slice
widths (T <= 64 and T > 64), plus the mixer wrapped around the tiny layer.

Bars (fp32 arithmetic throughout, fp64 oracle): coefficients within 2e-5
absolute; reduced rows and expanded streams within 2e-5 of the row's
largest magnitude; the bf16 copy is the GPU's fp32 row rounded to nearest
even, bit for bit; the expand step alone, fed the oracle's coefficients,
within 1e-6; in place equals out of place bit for bit."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from bit_quantized_routed_router_amd import ds4moe as D
from bit_quantized_routed_router_amd import synthetic as S
from tests.gpu_helpers import SeededLayer, dev, host, rel_err_rows

pytestmark = pytest.mark.gpu

COEF_TOL = 2e-5
ROW_TOL = 2e-5


def bf16_rne_bits(a: np.ndarray) -> np.ndarray:
    return S.f32_to_bf16_bits(np.ascontiguousarray(a, dtype=np.float32))


class Mixer:
    def __init__(self, d, T, variant=0):
        self.d, self.T = d, T
        self.X, self.phi, self.bias, self.alpha, self.y = S.gen_hc(d, T, variant=variant)
        self.H = D.Hc(d, dev(self.phi), dev(self.bias), self.alpha, S.HC_EPS, S.HC_SINKHORN_ITERS)
        self.Xd = dev(self.X)

    def oracle_pre(self):
        return O.hc_pre(self.X, self.phi, self.bias, self.alpha, S.HC_EPS, S.HC_SINKHORN_ITERS)

    def pre(self, bf16=True):
        T, d = self.T, self.d
        coef = torch.empty((T, 24), dtype=torch.float32, device="cuda")
        xo = torch.empty((T, d), dtype=torch.float32, device="cuda")
        xb = torch.empty((T, d), dtype=torch.int16, device="cuda") if bf16 else None
        ws, n = self.H.workspace(T)
        D.hc_pre(self.H.desc, self.Xd, T, coef, xo, xb, ws, n)
        torch.cuda.synchronize()
        return host(coef), host(xo), None if xb is None else host(xb, np.uint16)

    def post(self, coef, y, inplace=False):
        T, d = self.T, self.d
        c = dev(np.ascontiguousarray(coef, dtype=np.float32))
        yd = dev(np.ascontiguousarray(y, dtype=np.float32))
        if inplace:
            out = self.Xd.clone()
            D.hc_post(self.H.desc, out, yd, c, T, out)
        else:
            out = torch.empty((T, 4, d), dtype=torch.float32, device="cuda")
            D.hc_post(self.H.desc, self.Xd, yd, c, T, out)
        torch.cuda.synchronize()
        return host(out)


def check_pre(m: Mixer, label: str):
    cref, xref = m.oracle_pre()
    coef, xo, xb = m.pre()
    cerr = float(np.abs(coef - cref).max())
    xerr = rel_err_rows(xo, xref)
    print(f"{label}: coef abs err {cerr:.2e}, x_in rel err {xerr:.2e}")
    assert cerr <= COEF_TOL, cerr
    assert xerr <= ROW_TOL, xerr
    assert np.array_equal(xb, bf16_rne_bits(xo))
    M = coef[:, 8:].reshape(-1, 4, 4)
    assert np.allclose(M.sum(axis=1), 1.0, atol=1e-5)  # columns of every mixer
    return cref, coef


@pytest.mark.parametrize("T", [1, 3, 16, 17, 40, 64, 65, 100])
def test_hc_small_width(T):
    m = Mixer(256, T, variant=T)
    cref, coef = check_pre(m, f"hc d=256 T={T}")
    got = m.post(coef, m.y)
    ref = O.hc_post(m.X, m.y, cref)
    err = rel_err_rows(got.reshape(T * 4, -1), ref.reshape(T * 4, -1))
    print(f"hc d=256 T={T} expand rel err {err:.2e}")
    assert err <= ROW_TOL


@pytest.mark.parametrize("T", [1, 4, 16])
def test_hc_decode_shape(T):
    m = Mixer(4096, T, variant=100 + T)
    cref, coef = check_pre(m, f"hc d=4096 T={T}")
    got = m.post(coef, m.y)
    ref = O.hc_post(m.X, m.y, cref)
    assert rel_err_rows(got.reshape(T * 4, -1), ref.reshape(T * 4, -1)) <= ROW_TOL


def test_hc_prefill_shape():
    T = 2048
    m = Mixer(4096, T, variant=7)
    cref, coef = check_pre(m, "hc d=4096 T=2048")
    got = m.post(coef, m.y)
    ref = O.hc_post(m.X, m.y, cref)
    assert rel_err_rows(got.reshape(T * 4, -1), ref.reshape(T * 4, -1)) <= ROW_TOL


def test_hc_post_alone_with_oracle_coefficients():
    m = Mixer(4096, 8, variant=3)
    cref, _ = m.oracle_pre()
    got = m.post(cref, m.y)
    ref = O.hc_post(m.X, m.y, cref.astype(np.float32).astype(np.float64))
    err = rel_err_rows(got.reshape(32, -1), ref.reshape(32, -1))
    print(f"expand alone rel err {err:.2e}")
    assert err <= 1e-6


def test_hc_post_in_place_equals_out_of_place():
    m = Mixer(512, 33, variant=5)
    coef, _, _ = m.pre()
    a = m.post(coef, m.y)
    b = m.post(coef, m.y, inplace=True)
    assert np.array_equal(a, b)


def test_hc_pre_optional_outputs_and_repeat():
    m = Mixer(1024, 5, variant=9)
    c1, x1, b1 = m.pre(bf16=True)
    c2, x2, b2 = m.pre(bf16=False)
    assert np.array_equal(c1, c2) and np.array_equal(x1, x2)
    # bf16 only
    T, d = m.T, m.d
    coef = torch.empty((T, 24), dtype=torch.float32, device="cuda")
    xb = torch.empty((T, d), dtype=torch.int16, device="cuda")
    ws, n = m.H.workspace(T)
    D.hc_pre(m.H.desc, m.Xd, T, coef, None, xb, ws, n)
    torch.cuda.synchronize()
    assert np.array_equal(host(xb, np.uint16), b1) and np.array_equal(host(coef), c1)


def test_hc_around_tiny_layer():
    """Mixer, layer, mixer: hc_pre's fp32 row feeds the tiny layer (fp32 x),
    its y feeds hc_post; the oracle runs the same chain in fp64 (its reduced
    row rounded to fp32 as the layer's input).  Routing exact, streams within
    the layer's 2e-3 bar."""
    L = SeededLayer(S.CONFIGS["tiny"], device_quantize=False)
    T, d = 12, L.cfg.d
    for variant in range(20):  # first seeded draw whose routing has a clear top-k margin
        m = Mixer(d, T, variant=200 + variant)
        cref, xref = m.oracle_pre()
        x32 = xref.astype(np.float32)
        r = L.oracle.route(x32, "f32")
        if O.topk_gap(r["logits"], L.cfg.k).min() > 1e-3:
            break
    else:
        pytest.fail("no seeded draw with a clear top-k margin")
    ref_layer = L.oracle.forward(x32, "f32")
    Xref = O.hc_post(m.X, ref_layer["y64"], cref)
    coef, xo, _ = m.pre()
    for mode in (D.MODE_DECODE, D.MODE_PREFILL):
        got = L.forward(xo, mode)
        assert np.array_equal(got["idx"], ref_layer["idx"])
        out = m.post(coef, got["y"])
        err = rel_err_rows(out.reshape(T * 4, -1), Xref.reshape(T * 4, -1))
        print(f"mixer around tiny layer mode={mode}: rel err {err:.2e}")
        assert err <= 2e-3
