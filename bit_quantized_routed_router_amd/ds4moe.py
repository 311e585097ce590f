"""Python binding of the ds4moe C ABI (include/ds4moe.h).

Argument marshalling only: every computation runs in the HIP library
libds4moe.so built next to this file.  PyTorch tensors supply device memory
and the current stream; the C functions see plain pointers and sizes.  The
module refuses to work without the built library (no CPU fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libds4moe.so")

OK, EINVAL, ESHAPE, EALIGN, EWORKSPACE, EHIP, EUNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
FMT_F16, FMT_CB2, FMT_Q2K, FMT_MXFP4, FMT_Q4K = 0, 1, 2, 3, 4
EXPERTS_CB2_Q2K, EXPERTS_MXFP4, EXPERTS_Q4K = 0, 1, 2
DT_F32, DT_BF16 = 0, 1
MODE_DECODE, MODE_PREFILL, MODE_ROUTE = 0, 1, 2
DECODE_MAX_T = 64


class Ds4moeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {strerror(status)} (status {status})")
        self.status = status


class LayerDesc(ctypes.Structure):
    """Mirror of ds4moe_layer."""
    _fields_ = [
        ("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("d_ff", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32),
        ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
        ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p), ("sh_down", ctypes.c_void_p),
        ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
        ("expert_fmt", ctypes.c_int32),
    ]


class HcDesc(ctypes.Structure):
    """Mirror of ds4moe_hc."""
    _fields_ = [
        ("n_streams", ctypes.c_int32), ("d_model", ctypes.c_int32), ("sinkhorn_iters", ctypes.c_int32),
        ("eps", ctypes.c_float), ("alpha_pre", ctypes.c_float), ("alpha_post", ctypes.c_float),
        ("alpha_res", ctypes.c_float), ("phi", ctypes.c_void_p), ("bias", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_routed_router_amd.build_lib`")
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        LP = ctypes.POINTER(LayerDesc)
        L.ds4moe_packed_bytes.restype = SZ
        L.ds4moe_packed_bytes.argtypes = [I32, I64, I64]
        L.ds4moe_quantize.restype = I32
        L.ds4moe_quantize.argtypes = [I32, P, I64, I64, P, P]
        L.ds4moe_dequantize.restype = I32
        L.ds4moe_dequantize.argtypes = [I32, P, I64, I64, P, P]
        L.ds4moe_workspace_bytes.restype = SZ
        L.ds4moe_workspace_bytes.argtypes = [LP, I64, I32]
        L.ds4moe_workspace_init.restype = I32
        L.ds4moe_workspace_init.argtypes = [P, SZ, P]
        L.ds4moe_route.restype = I32
        L.ds4moe_route.argtypes = [LP, P, I32, I64, P, P, P, P, P, P, SZ, P]
        L.ds4moe_forward_decode.restype = I32
        L.ds4moe_forward_decode.argtypes = [LP, P, I32, I64, P, P, P, P, SZ, P]
        L.ds4moe_forward_decode_static.restype = I32
        L.ds4moe_forward_decode_static.argtypes = [LP, P, I32, I64, P, P, P, P]
        L.ds4moe_forward_prefill.restype = I32
        L.ds4moe_forward_prefill.argtypes = [LP, P, I32, I64, P, P, P, P, P, SZ, P]
        HP = ctypes.POINTER(HcDesc)
        L.ds4moe_hc_workspace_bytes.restype = SZ
        L.ds4moe_hc_workspace_bytes.argtypes = [HP, I64]
        L.ds4moe_hc_pre.restype = I32
        L.ds4moe_hc_pre.argtypes = [HP, P, I64, P, P, P, P, SZ, P]
        L.ds4moe_hc_post.restype = I32
        L.ds4moe_hc_post.argtypes = [HP, P, P, P, I64, P, P]
        L.ds4moe_strerror.restype = ctypes.c_char_p
        L.ds4moe_strerror.argtypes = [I32]
        L.ds4moe_trace_enable.restype = I32
        L.ds4moe_trace_enable.argtypes = [I32]
        L.ds4moe_trace_read.restype = I32
        L.ds4moe_trace_read.argtypes = [P, SZ, P, P, I32, I32]
        L.ds4moe_grid_levels.restype = None
        L.ds4moe_grid_levels.argtypes = [P]
        _lib = L
    return _lib


EXPORTS = ["ds4moe_packed_bytes", "ds4moe_quantize", "ds4moe_dequantize", "ds4moe_workspace_bytes",
           "ds4moe_workspace_init",
           "ds4moe_route", "ds4moe_forward_decode", "ds4moe_forward_decode_static", "ds4moe_forward_prefill", "ds4moe_strerror",
           "ds4moe_grid_levels", "ds4moe_trace_enable", "ds4moe_trace_read",
           "ds4moe_hc_workspace_bytes", "ds4moe_hc_pre", "ds4moe_hc_post"]


def strerror(status: int) -> str:
    return lib().ds4moe_strerror(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != OK:
        raise Ds4moeError(status, what)


def packed_bytes(fmt: int, rows: int, cols: int) -> int:
    return int(lib().ds4moe_packed_bytes(fmt, rows, cols))


def quantize(fmt: int, w, rows: int, cols: int, packed, stream=None) -> None:
    _check(lib().ds4moe_quantize(fmt, _ptr(w), rows, cols, _ptr(packed), _stream(stream)), "ds4moe_quantize")


def dequantize(fmt: int, packed, rows: int, cols: int, w, stream=None) -> None:
    _check(lib().ds4moe_dequantize(fmt, _ptr(packed), rows, cols, _ptr(w), _stream(stream)), "ds4moe_dequantize")


def workspace_bytes(desc: LayerDesc, T: int, mode: int) -> int:
    return int(lib().ds4moe_workspace_bytes(ctypes.byref(desc), T, mode))


def workspace_init(ws, nbytes: int, stream=None) -> None:
    """Zero a new workspace (required once before its first forward call)."""
    _check(lib().ds4moe_workspace_init(_ptr(ws), int(nbytes), _stream(stream)), "ds4moe_workspace_init")


def route(desc, x, x_dtype, T, topk_idx, topk_w, counts, offsets, perm, ws, ws_bytes, stream=None) -> None:
    _check(lib().ds4moe_route(ctypes.byref(desc), _ptr(x), x_dtype, T, _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
                              _ptr(offsets), _ptr(perm), _ptr(ws), ws_bytes, _stream(stream)), "ds4moe_route")


def forward_decode(desc, x, x_dtype, T, y, topk_idx_out, topk_w_out, ws, ws_bytes, stream=None) -> None:
    _check(lib().ds4moe_forward_decode(ctypes.byref(desc), _ptr(x), x_dtype, T, _ptr(y), _ptr(topk_idx_out),
                                       _ptr(topk_w_out), _ptr(ws), ws_bytes, _stream(stream)), "ds4moe_forward_decode")


STATIC_SCRATCH_BYTES = 4 << 20


def forward_decode_static(desc, x, x_dtype, T, y, topk_idx_out, topk_w_out, stream=None) -> None:
    """forward_decode on the library's own device array (no workspace)."""
    _check(lib().ds4moe_forward_decode_static(ctypes.byref(desc), _ptr(x), x_dtype, T, _ptr(y), _ptr(topk_idx_out),
                                              _ptr(topk_w_out), _stream(stream)), "ds4moe_forward_decode_static")


def forward_prefill(desc, x, x_dtype, T, y, topk_idx_out, topk_w_out, perm_out, ws, ws_bytes, stream=None) -> None:
    _check(lib().ds4moe_forward_prefill(ctypes.byref(desc), _ptr(x), x_dtype, T, _ptr(y), _ptr(topk_idx_out),
                                        _ptr(topk_w_out), _ptr(perm_out), _ptr(ws), ws_bytes, _stream(stream)),
           "ds4moe_forward_prefill")


def hc_workspace_bytes(desc: HcDesc, T: int) -> int:
    return int(lib().ds4moe_hc_workspace_bytes(ctypes.byref(desc), T))


def hc_pre(desc, X, T, coef, x_out, x_bf16, ws, ws_bytes, stream=None) -> None:
    _check(lib().ds4moe_hc_pre(ctypes.byref(desc), _ptr(X), T, _ptr(coef), _ptr(x_out), _ptr(x_bf16), _ptr(ws),
                               ws_bytes, _stream(stream)), "ds4moe_hc_pre")


def hc_post(desc, X, y, coef, T, X_out, stream=None) -> None:
    _check(lib().ds4moe_hc_post(ctypes.byref(desc), _ptr(X), _ptr(y), _ptr(coef), T, _ptr(X_out), _stream(stream)),
           "ds4moe_hc_post")


class Hc:
    """Device tensors of one hyper-connection mixer plus its ds4moe_hc
    descriptor: phi float32 [2n + n*n, n*d], bias float32 [2n + n*n] (CUDA
    tensors), alpha (pre, post, res)."""

    def __init__(self, d, phi, bias, alpha, eps=1e-6, iters=20, n=4):
        self.tensors = dict(phi=phi, bias=bias)
        self.d, self.n = d, n
        a = [float(v) for v in alpha]
        self.desc = HcDesc(n, d, iters, float(eps), a[0], a[1], a[2], _ptr(phi), _ptr(bias))

    def workspace(self, T: int):
        n = hc_workspace_bytes(self.desc, T)
        if n == 0:
            raise Ds4moeError(ESHAPE, "ds4moe_hc_workspace_bytes")
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        workspace_init(ws, n)
        return ws, n


def trace_enable(on: bool) -> None:
    lib().ds4moe_trace_enable(1 if on else 0)


def trace_read(reset: bool = True) -> dict:
    """{kernel name: (total ms, launches)} accumulated since the last reset."""
    cap = 64
    names = ctypes.create_string_buffer(8192)
    ms = (ctypes.c_double * cap)()
    cnt = (ctypes.c_longlong * cap)()
    n = lib().ds4moe_trace_read(names, 8192, ctypes.cast(ms, ctypes.c_void_p), ctypes.cast(cnt, ctypes.c_void_p),
                                cap, 1 if reset else 0)
    if n < 0:
        raise Ds4moeError(n, "ds4moe_trace_read")
    keys = names.value.decode().split("\n")[:min(n, cap)]
    return {k: (ms[i], cnt[i]) for i, k in enumerate(keys)}


def grid_levels():
    import numpy as np
    out = np.zeros((256, 8), dtype=np.uint8)
    lib().ds4moe_grid_levels(out.ctypes.data_as(ctypes.c_void_p))
    return out


class Layer:
    """Device tensors of one layer plus its ds4moe_layer descriptor.

    router_w, sh_gate, sh_up, sh_down: binary16 bit patterns (int16/uint16 or
    float16 CUDA tensors); gate/up/down: uint8 CUDA tensors of E packed
    matrices each; router_bias: float32 CUDA tensor or None; expert_fmt:
    EXPERTS_CB2_Q2K, EXPERTS_MXFP4 or EXPERTS_Q4K.
    """

    def __init__(self, d, E, k, f, fs, router_w, router_bias, sh_gate, sh_up, sh_down, gate, up, down,
                 expert_fmt=EXPERTS_CB2_Q2K):
        self.tensors = dict(router_w=router_w, router_bias=router_bias, sh_gate=sh_gate, sh_up=sh_up,
                            sh_down=sh_down, gate=gate, up=up, down=down)
        self.d, self.E, self.k, self.f, self.fs = d, E, k, f, fs
        self.expert_fmt = expert_fmt
        self.desc = LayerDesc(d, E, k, f, fs, _ptr(router_w), _ptr(router_bias), _ptr(sh_gate), _ptr(sh_up),
                              _ptr(sh_down), _ptr(gate), _ptr(up), _ptr(down), expert_fmt)

    def with_experts(self, gate, up, down) -> "Layer":
        t = dict(self.tensors)
        return Layer(self.d, self.E, self.k, self.f, self.fs, t["router_w"], t["router_bias"], t["sh_gate"],
                     t["sh_up"], t["sh_down"], gate, up, down, self.expert_fmt)

    def workspace(self, T: int, mode: int):
        n = workspace_bytes(self.desc, T, mode)
        if n == 0:
            raise Ds4moeError(ESHAPE, "ds4moe_workspace_bytes")
        ws = torch.empty(n + 256, dtype=torch.uint8, device="cuda")
        workspace_init(ws, n)
        return ws, n
