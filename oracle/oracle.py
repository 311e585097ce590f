"""ds4moe CPU oracle, Python side -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this module; the product path never does.  It loads the
plain C oracle (liboracle.so, built with gcc from ds4moe_oracle.c) through
ctypes and composes the layer from its steps in fp64:

  route    logits = x . Wr^T (+ bias)            F16 router (DS4 (DwarfStar 4)
           k largest logits, ascending index      wiki note, "Key Techniques")
           w = softmax over the selected
  group    counts, offsets, perm, inv
  experts  h = silu(G x) * (U x), out = D h       gate/up CB2, down Q2K
  shared   ys = Wsd (silu(Wsg x) * (Wsu x))       F16
  combine  y = ys + sum_j w_j out_j, rounded once to float32

Readings where the pages are silent (score function, weight normalisation,
slot order, activation) are stated in ds4moe_oracle.c next to each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ds4moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
QK = 256

GCC_CMD = ["gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", _LIB_PATH, _SRC, "-lm"]


def build() -> str:
    subprocess.check_call(GCC_CMD)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f64_to_f16.restype = ctypes.c_uint16
        L.orc_f64_to_f16.argtypes = [ctypes.c_double]
        L.orc_bf16_to_f64.restype = ctypes.c_double
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_splitmix64.restype = ctypes.c_uint64
        L.orc_splitmix64.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
        L.orc_grid_levels.argtypes = [P]
        L.orc_cb2_dequantize.argtypes = [P, P, I64, I64, P]
        L.orc_cb2_quantize.argtypes = [P, I64, I64, P, P]
        L.orc_q2k_dequantize.argtypes = [P, P, P, I64, I64, P]
        L.orc_q2k_quantize.argtypes = [P, I64, I64, P, P, P]
        L.orc_cb2_matmul.argtypes = [P, P, I64, I64, P, I64, P]
        L.orc_q2k_matmul.argtypes = [P, P, P, I64, I64, P, I64, P]
        L.orc_f16_matmul.argtypes = [P, I64, I64, P, I64, P]
        L.orc_router_logits.argtypes = [P, I64, I64, P, I64, P, P]
        L.orc_topk.argtypes = [P, I64, I64, ctypes.c_int, P, P]
        L.orc_permute.argtypes = [P, I64, ctypes.c_int, I64, P, P, P, P]
        L.orc_swiglu.argtypes = [P, P, I64, P]
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_int]
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [ctypes.c_int]
        L.orc_mx4_dequantize.argtypes = [P, P, I64, I64, P]
        L.orc_mx4_quantize.argtypes = [P, I64, I64, P, P]
        L.orc_mx4_matmul.argtypes = [P, P, I64, I64, P, I64, P]
        L.orc_q4k_dequantize.argtypes = [P, P, P, I64, I64, P]
        L.orc_q4k_quantize.argtypes = [P, I64, I64, P, P, P]
        L.orc_sinkhorn.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
        L.orc_hc_pre.argtypes = [P, I64, ctypes.c_int, I64, P, P, P, ctypes.c_double, ctypes.c_int, P, P]
        L.orc_hc_post.argtypes = [P, P, P, I64, ctypes.c_int, I64, P]
        L.orc_q4k_matmul.argtypes = [P, P, P, I64, I64, P, I64, P]
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from the calling thread on."""
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ---------------------------------------------------------------- scalars
def f16_to_f64(bits: int) -> float:
    return lib().orc_f16_to_f64(int(bits))


def f64_to_f16(v: float) -> int:
    return lib().orc_f64_to_f16(float(v))


def bf16_to_f64(bits: int) -> float:
    return lib().orc_bf16_to_f64(int(bits))


def splitmix64_sequence(seed: int, n: int) -> list[int]:
    st = ctypes.c_uint64(seed)
    return [lib().orc_splitmix64(ctypes.byref(st)) for _ in range(n)]


def grid_levels() -> np.ndarray:
    out = np.zeros((256, 8), dtype=np.uint8)
    lib().orc_grid_levels(_p(out))
    return out


# ---------------------------------------------------------------- packed matrices
# A packed matrix is one byte buffer holding its planes back to back:
#   CB2 [rows, cols]: codes rows*nb*64 B, then d (binary16) rows*nb*2 B
#   Q2K [rows, cols]: codes rows*nb*64 B, subscales rows*nb*16 B,
#                     then (d, dmin) binary16 pairs rows*nb*4 B
def cb2_bytes(rows: int, cols: int) -> int:
    return rows * (cols // QK) * 66


def q2k_bytes(rows: int, cols: int) -> int:
    return rows * (cols // QK) * 84


def q4k_bytes(rows: int, cols: int) -> int:
    return rows * (cols // QK) * 144


def q4k_planes(packed: np.ndarray, rows: int, cols: int):
    n = rows * (cols // QK)
    return packed[: n * 128], packed[n * 128: n * 140], packed[n * 140: n * 144].view(np.uint16)


def mx4_bytes(rows: int, cols: int) -> int:
    return rows * cols // 2 + rows * cols // 32


def cb2_planes(packed: np.ndarray, rows: int, cols: int):
    nb = cols // QK
    n = rows * nb
    codes = packed[: n * 64]
    d = packed[n * 64: n * 66].view(np.uint16)
    return codes, d


def q2k_planes(packed: np.ndarray, rows: int, cols: int):
    nb = cols // QK
    n = rows * nb
    codes = packed[: n * 64]
    sub = packed[n * 64: n * 80]
    sup = packed[n * 80: n * 84].view(np.uint16)
    return codes, sub, sup


def mx4_planes(packed: np.ndarray, rows: int, cols: int):
    n = rows * cols
    return packed[: n // 2], packed[n // 2: n // 2 + n // 32]


def _check(rows, cols):
    if cols % QK != 0 or rows < 0:
        raise ValueError("cols must be a multiple of 256")


def cb2_quantize(w: np.ndarray) -> np.ndarray:
    rows, cols = w.shape
    _check(rows, cols)
    w = np.ascontiguousarray(w, dtype=np.float32)
    packed = np.zeros(cb2_bytes(rows, cols), dtype=np.uint8)
    codes, d = cb2_planes(packed, rows, cols)
    lib().orc_cb2_quantize(_p(w), rows, cols, _p(codes), _p(d))
    return packed


def cb2_dequantize(packed: np.ndarray, rows: int, cols: int) -> np.ndarray:
    _check(rows, cols)
    codes, d = cb2_planes(np.ascontiguousarray(packed), rows, cols)
    out = np.zeros((rows, cols), dtype=np.float32)
    lib().orc_cb2_dequantize(_p(codes), _p(d), rows, cols, _p(out))
    return out


def q2k_quantize(w: np.ndarray) -> np.ndarray:
    rows, cols = w.shape
    _check(rows, cols)
    w = np.ascontiguousarray(w, dtype=np.float32)
    packed = np.zeros(q2k_bytes(rows, cols), dtype=np.uint8)
    codes, sub, sup = q2k_planes(packed, rows, cols)
    lib().orc_q2k_quantize(_p(w), rows, cols, _p(codes), _p(sub), _p(sup))
    return packed


def q2k_dequantize(packed: np.ndarray, rows: int, cols: int) -> np.ndarray:
    _check(rows, cols)
    codes, sub, sup = q2k_planes(np.ascontiguousarray(packed), rows, cols)
    out = np.zeros((rows, cols), dtype=np.float32)
    lib().orc_q2k_dequantize(_p(codes), _p(sub), _p(sup), rows, cols, _p(out))
    return out


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e8m0_value(code: int) -> float:
    return lib().orc_e8m0_value(int(code))


def q4k_quantize(w: np.ndarray) -> np.ndarray:
    rows, cols = w.shape
    _check(rows, cols)
    w = np.ascontiguousarray(w, dtype=np.float32)
    packed = np.zeros(q4k_bytes(rows, cols), dtype=np.uint8)
    codes, sc, sup = q4k_planes(packed, rows, cols)
    lib().orc_q4k_quantize(_p(w), rows, cols, _p(codes), _p(sc), _p(sup))
    return packed


def q4k_dequantize(packed: np.ndarray, rows: int, cols: int) -> np.ndarray:
    _check(rows, cols)
    codes, sc, sup = q4k_planes(np.ascontiguousarray(packed), rows, cols)
    out = np.zeros((rows, cols), dtype=np.float32)
    lib().orc_q4k_dequantize(_p(codes), _p(sc), _p(sup), rows, cols, _p(out))
    return out


def mx4_quantize(w: np.ndarray) -> np.ndarray:
    rows, cols = w.shape
    _check(rows, cols)
    w = np.ascontiguousarray(w, dtype=np.float32)
    packed = np.zeros(mx4_bytes(rows, cols), dtype=np.uint8)
    codes, sc = mx4_planes(packed, rows, cols)
    lib().orc_mx4_quantize(_p(w), rows, cols, _p(codes), _p(sc))
    return packed


def mx4_dequantize(packed: np.ndarray, rows: int, cols: int) -> np.ndarray:
    _check(rows, cols)
    codes, sc = mx4_planes(np.ascontiguousarray(packed), rows, cols)
    out = np.zeros((rows, cols), dtype=np.float32)
    lib().orc_mx4_dequantize(_p(codes), _p(sc), rows, cols, _p(out))
    return out


# ---------------------------------------------------------------- products (fp64)
def cb2_matmul(packed, rows, cols, X: np.ndarray) -> np.ndarray:
    X = np.ascontiguousarray(X, dtype=np.float64)
    n = X.shape[0]
    codes, d = cb2_planes(packed, rows, cols)
    Y = np.zeros((n, rows), dtype=np.float64)
    lib().orc_cb2_matmul(_p(codes), _p(d), rows, cols, _p(X), n, _p(Y))
    return Y


def q2k_matmul(packed, rows, cols, X: np.ndarray) -> np.ndarray:
    X = np.ascontiguousarray(X, dtype=np.float64)
    n = X.shape[0]
    codes, sub, sup = q2k_planes(packed, rows, cols)
    Y = np.zeros((n, rows), dtype=np.float64)
    lib().orc_q2k_matmul(_p(codes), _p(sub), _p(sup), rows, cols, _p(X), n, _p(Y))
    return Y


def q4k_matmul(packed, rows, cols, X: np.ndarray) -> np.ndarray:
    X = np.ascontiguousarray(X, dtype=np.float64)
    n = X.shape[0]
    codes, sc, sup = q4k_planes(packed, rows, cols)
    Y = np.zeros((n, rows), dtype=np.float64)
    lib().orc_q4k_matmul(_p(codes), _p(sc), _p(sup), rows, cols, _p(X), n, _p(Y))
    return Y


def mx4_matmul(packed, rows, cols, X: np.ndarray) -> np.ndarray:
    X = np.ascontiguousarray(X, dtype=np.float64)
    n = X.shape[0]
    codes, sc = mx4_planes(packed, rows, cols)
    Y = np.zeros((n, rows), dtype=np.float64)
    lib().orc_mx4_matmul(_p(codes), _p(sc), rows, cols, _p(X), n, _p(Y))
    return Y


def f16_matmul(w_bits: np.ndarray, X: np.ndarray) -> np.ndarray:
    rows, cols = w_bits.shape
    w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16)
    X = np.ascontiguousarray(X, dtype=np.float64)
    n = X.shape[0]
    Y = np.zeros((n, rows), dtype=np.float64)
    lib().orc_f16_matmul(_p(w_bits), rows, cols, _p(X), n, _p(Y))
    return Y


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    h = np.zeros_like(g)
    lib().orc_swiglu(_p(g), _p(u), g.size, _p(h))
    return h


# ---------------------------------------------------------------- routing
# ---------------------------------------------------------------- HC mixer
def sinkhorn(Z: np.ndarray, iters: int) -> np.ndarray:
    """exp(Z) for an [n, n] Z after `iters` Sinkhorn iterations (rows, then
    columns, each divided by its sum)."""
    Z = np.ascontiguousarray(Z, dtype=np.float64)
    n = Z.shape[0]
    A = np.empty((n, n), dtype=np.float64)
    lib().orc_sinkhorn(_p(Z), n, iters, _p(A))
    return A


def hc_pre(X: np.ndarray, phi: np.ndarray, bias: np.ndarray, alpha, eps: float, iters: int):
    """Coefficients and reduced rows of the hyper-connection mixer.
    X [T, n, d]; phi [2n + n*n, n*d]; bias [2n + n*n]; alpha (pre, post, res).
    Returns coef [T, 2n + n*n] (pre, post, M row-major) and x_in [T, d]."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    T, n, d = X.shape
    no = 2 * n + n * n
    phi = np.ascontiguousarray(phi, dtype=np.float64)
    bias = np.ascontiguousarray(bias, dtype=np.float64)
    assert phi.shape == (no, n * d) and bias.shape == (no,)
    a = np.ascontiguousarray(alpha, dtype=np.float64)
    coef = np.empty((T, no), dtype=np.float64)
    xin = np.empty((T, d), dtype=np.float64)
    lib().orc_hc_pre(_p(X), T, n, d, _p(phi), _p(bias), _p(a), float(eps), iters, _p(coef), _p(xin))
    return coef, xin


def hc_post(X: np.ndarray, y: np.ndarray, coef: np.ndarray) -> np.ndarray:
    """Expanded streams X' [T, n, d] = M X + post y per token."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    T, n, d = X.shape
    y = np.ascontiguousarray(y, dtype=np.float64)
    coef = np.ascontiguousarray(coef, dtype=np.float64)
    assert y.shape == (T, d) and coef.shape == (T, 2 * n + n * n)
    out = np.empty_like(X)
    lib().orc_hc_post(_p(X), _p(y), _p(coef), T, n, d, _p(out))
    return out


def x_to_f64(x: np.ndarray, x_dtype: str) -> np.ndarray:
    """Activations to fp64, exactly: float32 values or bfloat16 bits."""
    if x_dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if x_dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    raise ValueError(x_dtype)


def router_logits(X: np.ndarray, wr_bits: np.ndarray, bias) -> np.ndarray:
    X = np.ascontiguousarray(X, dtype=np.float64)
    T, d = X.shape
    E = wr_bits.shape[0]
    wr_bits = np.ascontiguousarray(wr_bits, dtype=np.uint16)
    out = np.zeros((T, E), dtype=np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    lib().orc_router_logits(_p(X), T, d, _p(wr_bits), E, None if b is None else _p(b), _p(out))
    return out


def topk(logits: np.ndarray, k: int):
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    T, E = logits.shape
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    lib().orc_topk(_p(logits), T, E, k, _p(idx), _p(w))
    return idx, w


def permute(idx: np.ndarray, E: int):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    perm = np.zeros(T * k, dtype=np.int32)
    inv = np.zeros(T * k, dtype=np.int32)
    lib().orc_permute(_p(idx), T, k, E, _p(counts), _p(offsets), _p(perm), _p(inv))
    return counts, offsets, perm, inv


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token: (k-th largest logit) - ((k+1)-th largest logit)."""
    s = -np.sort(-logits, axis=1)
    return s[:, k - 1] - s[:, k]


# ---------------------------------------------------------------- layer
class Layer:
    """One routed-MoE layer for the oracle.

    experts: callable e -> (gate_packed, up_packed, down_packed), or a dict.
    Packed matrices follow the plane layout above; router and shared weights
    are binary16 bit arrays.  expert_fmt: "cb2q2k" (CB2 gate/up, Q2K down),
    "mxfp4" (all three in MXFP4) or "q4k" (all three in Q4K).
    """

    def __init__(self, d, E, k, f, fs, router_bits, bias, sh_gate, sh_up, sh_down, experts, expert_fmt="cb2q2k"):
        self.d, self.E, self.k, self.f, self.fs = d, E, k, f, fs
        self.expert_fmt = expert_fmt
        self.router_bits, self.bias = router_bits, bias
        self.sh_gate, self.sh_up, self.sh_down = sh_gate, sh_up, sh_down
        self._experts = experts
        self._cache = {}

    def expert(self, e):
        if e not in self._cache:
            src = self._experts
            self._cache[e] = src[e] if isinstance(src, dict) else src(e)
        return self._cache[e]

    def route(self, x, x_dtype):
        X = x_to_f64(x, x_dtype)
        logits = router_logits(X, self.router_bits, self.bias)
        idx, w = topk(logits, self.k)
        counts, offsets, perm, inv = permute(idx, self.E)
        return dict(X=X, logits=logits, idx=idx, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv)

    def shared(self, X):
        g = f16_matmul(self.sh_gate, X)
        u = f16_matmul(self.sh_up, X)
        return f16_matmul(self.sh_down, swiglu(g, u))

    def expert_out(self, e, Xe):
        gp, up, dp = self.expert(e)
        if self.expert_fmt == "mxfp4":
            g = mx4_matmul(gp, self.f, self.d, Xe)
            u = mx4_matmul(up, self.f, self.d, Xe)
            return mx4_matmul(dp, self.d, self.f, swiglu(g, u))
        if self.expert_fmt == "q4k":
            g = q4k_matmul(gp, self.f, self.d, Xe)
            u = q4k_matmul(up, self.f, self.d, Xe)
            return q4k_matmul(dp, self.d, self.f, swiglu(g, u))
        g = cb2_matmul(gp, self.f, self.d, Xe)
        u = cb2_matmul(up, self.f, self.d, Xe)
        return q2k_matmul(dp, self.d, self.f, swiglu(g, u))

    def forward(self, x, x_dtype, tokens=None):
        """Full layer.  With `tokens`, y is computed only for those token rows
        (routing and grouping always cover every token)."""
        r = self.route(x, x_dtype)
        X, idx, w = r["X"], r["idx"], r["w"]
        T = X.shape[0]
        tok = np.arange(T) if tokens is None else np.asarray(tokens)
        out = np.zeros((len(tok), self.k, self.d), dtype=np.float64)
        pos = {int(t): i for i, t in enumerate(tok)}
        for e in np.unique(idx[tok]):
            rows = [(pos[int(t)], j) for t in tok for j in range(self.k) if idx[t, j] == e]
            Xe = np.stack([X[tok[i]] for i, _ in rows])
            Oe = self.expert_out(int(e), Xe)
            for n, (i, j) in enumerate(rows):
                out[i, j] = Oe[n]
        ys = self.shared(X[tok])
        y = ys.copy()
        for j in range(self.k):
            y += w[tok, j][:, None] * out[:, j, :]
        r.update(y=y.astype(np.float32), y64=y, tokens=tok, ys=ys)
        return r
