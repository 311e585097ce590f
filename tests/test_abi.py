"""Host-side checks of the C ABI (no device work): the library loads, exports
every function declared in include/ds4moe.h, sizes its buffers as the format
prescribes, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

from bit_quantized_routed_router_amd import ds4moe as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds4moe.h")

A = 0x10000  # stand-in device addresses: aligned, never dereferenced


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ds4moe_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = D.lib()
    names = header_functions()
    assert "ds4moe_forward_decode" in names and "ds4moe_quantize" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(D.EXPORTS)


def test_packed_sizes():
    assert D.packed_bytes(D.FMT_CB2, 2048, 4096) == 2048 * 16 * 66 == 2162688
    assert D.packed_bytes(D.FMT_Q2K, 4096, 2048) == 4096 * 8 * 84 == 2752512
    assert D.packed_bytes(D.FMT_F16, 3, 5) == 30
    assert D.packed_bytes(D.FMT_MXFP4, 2048, 4096) == 2048 * 4096 * 17 // 32 == 4456448
    assert D.packed_bytes(D.FMT_Q4K, 2048, 4096) == 2048 * 16 * 144 == 4718592
    assert D.packed_bytes(D.FMT_CB2, 4, 300) == 0
    assert D.packed_bytes(9, 4, 256) == 0


def desc(d=4096, E=256, k=6, f=2048, fs=2048, **ptr):
    p = dict(router_w=A, router_bias=None, sh_gate=A, sh_up=A, sh_down=A, gate=A, up=A, down=A)
    p.update(ptr)
    return D.LayerDesc(d, E, k, f, fs, p["router_w"], p["router_bias"], p["sh_gate"], p["sh_up"], p["sh_down"],
                       p["gate"], p["up"], p["down"])


def test_workspace_sizes():
    L = desc()
    dec = D.workspace_bytes(L, 1, D.MODE_DECODE)
    assert dec > 0 and dec % 256 == 0
    assert D.workspace_bytes(L, 64, D.MODE_DECODE) == D.workspace_bytes(L, 16, D.MODE_DECODE)
    pre = D.workspace_bytes(L, 2048, D.MODE_PREFILL)
    assert pre >= 2048 * 6 * 4096 * 4  # per-slot fp32 outputs
    assert D.workspace_bytes(L, 2048, D.MODE_ROUTE) < pre
    assert D.workspace_bytes(L, 0, D.MODE_DECODE) == 0
    assert D.workspace_bytes(desc(d=300), 1, D.MODE_DECODE) == 0
    assert D.workspace_bytes(L, 1, 7) == 0


def call_decode(L, x=A, dt=D.DT_BF16, T=1, y=A, ws=A * 16, nbytes=1 << 40):
    lib = D.lib()
    return lib.ds4moe_forward_decode(ctypes.byref(L) if L is not None else None, x, dt, T, y, None, None, ws,
                                     nbytes, None)


def test_forward_argument_errors():
    L = desc()
    assert call_decode(None) == D.EINVAL
    assert call_decode(desc(router_w=None)) == D.EINVAL
    assert call_decode(desc(d=4000)) == D.ESHAPE
    assert call_decode(desc(f=100)) == D.ESHAPE
    assert call_decode(desc(k=7, E=6)) == D.ESHAPE
    assert call_decode(desc(k=0)) == D.ESHAPE
    assert call_decode(desc(E=2000)) == D.ESHAPE
    assert call_decode(desc(gate=A + 4)) == D.EALIGN
    assert call_decode(desc(router_bias=A + 2)) == D.EALIGN
    bad = desc()
    bad.expert_fmt = 7
    assert call_decode(bad) == D.EINVAL
    assert call_decode(L, T=0) == D.ESHAPE
    assert call_decode(L, T=65) == D.ESHAPE
    assert call_decode(L, dt=5) == D.EINVAL
    assert call_decode(L, x=None) == D.EINVAL
    assert call_decode(L, y=None) == D.EINVAL
    assert call_decode(L, x=A + 8) == D.EALIGN
    assert call_decode(L, ws=A + 16) == D.EALIGN
    assert call_decode(L, nbytes=1024) == D.EWORKSPACE
    lib = D.lib()
    assert lib.ds4moe_forward_prefill(ctypes.byref(L), A, D.DT_BF16, 0, A, None, None, None, A, 1 << 40, None) == D.ESHAPE
    assert lib.ds4moe_forward_prefill(ctypes.byref(L), A, D.DT_BF16, 10**7, A, None, None, None, A, 1 << 40, None) == D.ESHAPE
    assert lib.ds4moe_route(ctypes.byref(L), A, D.DT_BF16, 4, None, A, None, None, None, A, 1 << 40, None) == D.EINVAL
    assert lib.ds4moe_route(ctypes.byref(L), A, D.DT_BF16, 4, A + 2, A, None, None, None, A, 1 << 40, None) == D.EALIGN


def test_static_decode_argument_errors():
    """The workspace-free decode rejects bad arguments, and shapes whose
    workspace exceeds its device array, before any HIP call."""
    lib = D.lib()

    def call(L, x=A, dt=D.DT_BF16, T=1, y=A):
        return lib.ds4moe_forward_decode_static(ctypes.byref(L) if L is not None else None, x, dt, T, y, None,
                                                None, None)

    big = desc(d=16384, E=1024, k=16, f=16384, fs=16384)
    assert D.workspace_bytes(big, 16, D.MODE_DECODE) > D.STATIC_SCRATCH_BYTES
    assert call(big, T=16) == D.EWORKSPACE
    assert D.workspace_bytes(desc(), 64, D.MODE_DECODE) <= D.STATIC_SCRATCH_BYTES
    assert call(None) == D.EINVAL
    assert call(desc(d=4000)) == D.ESHAPE
    assert call(desc(), T=0) == D.ESHAPE
    assert call(desc(), T=65) == D.ESHAPE
    assert call(desc(), dt=3) == D.EINVAL
    assert call(desc(), y=None) == D.EINVAL
    assert call(desc(), x=A + 2) == D.EALIGN


def test_header_static_scratch_size_matches_binding():
    src = open(HEADER).read()
    m = re.search(r"#define DS4MOE_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == D.STATIC_SCRATCH_BYTES


def test_codec_argument_errors():
    lib = D.lib()
    assert lib.ds4moe_quantize(7, A, 4, 256, A, None) == D.EINVAL
    assert lib.ds4moe_quantize(D.FMT_F16, A, 4, 256, A, None) == D.EINVAL
    assert lib.ds4moe_quantize(D.FMT_CB2, A, 4, 300, A, None) == D.ESHAPE
    assert lib.ds4moe_quantize(D.FMT_MXFP4, A, 4, 288, A, None) == D.ESHAPE
    assert lib.ds4moe_quantize(D.FMT_Q4K + 1, A, 4, 256, A, None) == D.EINVAL
    assert lib.ds4moe_quantize(D.FMT_CB2, A, -1, 256, A, None) == D.EINVAL
    assert lib.ds4moe_quantize(D.FMT_CB2, None, 4, 256, A, None) == D.EINVAL
    assert lib.ds4moe_quantize(D.FMT_Q2K, A + 4, 4, 256, A, None) == D.EALIGN
    assert lib.ds4moe_quantize(D.FMT_Q2K, A, 0, 256, None, None) == D.OK  # empty: nothing to do
    assert lib.ds4moe_dequantize(D.FMT_Q2K, A, 4, 257, A, None) == D.ESHAPE


def test_strerror_covers_codes():
    for c in (D.OK, D.EINVAL, D.ESHAPE, D.EALIGN, D.EWORKSPACE, D.EHIP, D.EUNSUPPORTED):
        assert D.strerror(c) and D.strerror(c) != "unknown status"
    assert D.strerror(12345) == "unknown status"


def test_grid_export_matches_oracle():
    from oracle import oracle as O
    assert (D.grid_levels() == O.grid_levels()).all()


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(D, "_lib", None)
    monkeypatch.setattr(D, "_LIB_PATH", "/nonexistent/libds4moe.so")
    with pytest.raises(RuntimeError):
        D.lib()


def hc_desc(**kw):
    v = dict(n_streams=4, d_model=4096, sinkhorn_iters=20, eps=1e-6, alpha_pre=1.0, alpha_post=1.0, alpha_res=1.0,
             phi=A, bias=A)
    v.update(kw)
    return D.HcDesc(**v)


def test_hc_workspace_sizes():
    lib = D.lib()
    # K-slices of 256 inputs (T <= 64) or 1024, 32 floats per (slice, token), then a 256-byte counter
    assert lib.ds4moe_hc_workspace_bytes(ctypes.byref(hc_desc()), 1) == 64 * 1 * 128 + 256
    assert lib.ds4moe_hc_workspace_bytes(ctypes.byref(hc_desc()), 64) == 64 * 64 * 128 + 256
    assert lib.ds4moe_hc_workspace_bytes(ctypes.byref(hc_desc()), 2048) == 16 * 2048 * 128 + 256
    assert lib.ds4moe_hc_workspace_bytes(ctypes.byref(hc_desc(d_model=256)), 65) == 8448 + 256  # 65 * 128 rounded up
    assert lib.ds4moe_hc_workspace_bytes(ctypes.byref(hc_desc()), 0) == 0
    assert lib.ds4moe_hc_workspace_bytes(ctypes.byref(hc_desc()), (1 << 20) + 1) == 0
    assert lib.ds4moe_hc_workspace_bytes(ctypes.byref(hc_desc(n_streams=2)), 1) == 0
    assert lib.ds4moe_hc_workspace_bytes(None, 1) == 0


def test_hc_argument_errors():
    lib = D.lib()
    big = 1 << 30
    pre = lambda h, X=A, T=1, coef=A, xo=A, xb=A, ws=A, n=big: lib.ds4moe_hc_pre(  # noqa: E731
        ctypes.byref(h), X, T, coef, xo, xb, ws, n, None)
    post = lambda h, X=A, y=A, coef=A, T=1, Xo=A: lib.ds4moe_hc_post(ctypes.byref(h), X, y, coef, T, Xo, None)  # noqa: E731
    h = hc_desc()
    assert pre(hc_desc(phi=None)) == D.EINVAL
    assert pre(hc_desc(bias=None)) == D.EINVAL
    assert pre(hc_desc(n_streams=0)) == D.EINVAL
    assert pre(hc_desc(n_streams=3)) == D.EUNSUPPORTED
    assert pre(hc_desc(d_model=300)) == D.ESHAPE
    assert pre(hc_desc(d_model=32768)) == D.ESHAPE
    assert pre(hc_desc(sinkhorn_iters=0)) == D.EINVAL
    assert pre(hc_desc(sinkhorn_iters=65)) == D.EINVAL
    assert pre(hc_desc(eps=-1.0)) == D.EINVAL
    assert pre(hc_desc(eps=float("nan"))) == D.EINVAL
    assert pre(hc_desc(alpha_res=float("inf"))) == D.EINVAL
    assert pre(hc_desc(phi=A + 4)) == D.EALIGN
    assert pre(hc_desc(bias=A + 2)) == D.EALIGN
    assert pre(h, X=None) == D.EINVAL
    assert pre(h, coef=None) == D.EINVAL
    assert pre(h, ws=None) == D.EINVAL
    assert pre(h, T=0) == D.ESHAPE
    assert pre(h, T=(1 << 20) + 1) == D.ESHAPE
    assert pre(h, X=A + 4) == D.EALIGN
    assert pre(h, xo=A + 8) == D.EALIGN
    assert pre(h, xb=A + 4) == D.EALIGN
    assert pre(h, ws=A + 16) == D.EALIGN
    assert pre(h, n=64 * 128 + 255) == D.EWORKSPACE
    assert post(hc_desc(n_streams=5)) == D.EUNSUPPORTED
    assert post(h, y=None) == D.EINVAL
    assert post(h, Xo=None) == D.EINVAL
    assert post(h, T=0) == D.ESHAPE
    assert post(h, coef=A + 4) == D.EALIGN
