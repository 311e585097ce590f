"""GPU parity of the codecs: ds4moe_dequantize bit-exact and ds4moe_quantize
byte-exact against the oracle."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from bit_quantized_routed_router_amd import ds4moe as D
from bit_quantized_routed_router_amd import synthetic as S
from tests.gpu_helpers import dev, host
from tests.test_oracle_formats import canonical_cb2, canonical_q2k

pytestmark = pytest.mark.gpu


def gpu_quant(fmt, w):
    rows, cols = w.shape
    out = torch.zeros(D.packed_bytes(fmt, rows, cols), dtype=torch.uint8, device="cuda")
    D.quantize(fmt, dev(w), rows, cols, out)
    torch.cuda.synchronize()
    return host(out)


def gpu_dequant(fmt, packed, rows, cols):
    out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    D.dequantize(fmt, dev(packed), rows, cols, out)
    torch.cuda.synchronize()
    return host(out)


def test_grid_matches_oracle():
    assert np.array_equal(D.grid_levels(), O.grid_levels())


@pytest.mark.parametrize("rows,cols,scale", [(1, 256, 0.02), (37, 512, 0.02), (64, 4096, 0.02), (5, 768, 30.0)])
def test_quantize_byte_exact(rows, cols, scale):
    w = (np.random.default_rng(rows * cols).standard_normal((rows, cols)) * scale).astype(np.float32)
    assert np.array_equal(gpu_quant(D.FMT_CB2, w), O.cb2_quantize(w))
    assert np.array_equal(gpu_quant(D.FMT_Q2K, w), O.q2k_quantize(w))


def test_quantize_edge_blocks_byte_exact():
    x = np.zeros((6, 256), dtype=np.float32)
    x[1, 17] = 0.5                       # single spike
    x[2, :] = 1e-9                       # d underflows
    x[3, 5], x[3, 6] = 3e38, -3e38       # d clamps at 65504
    x[4, :] = -0.01                      # all negative
    x[5, ::2] = 0.03                     # sub-blocks with exact ties
    x[5, 1::2] = -0.03
    assert np.array_equal(gpu_quant(D.FMT_CB2, x), O.cb2_quantize(x))
    assert np.array_equal(gpu_quant(D.FMT_Q2K, x), O.q2k_quantize(x))


def test_quantize_canonical_round_trip():
    rng = np.random.default_rng(9)
    cb = canonical_cb2(rng, 32)
    w = O.cb2_dequantize(cb, 32, 256)
    assert np.array_equal(gpu_quant(D.FMT_CB2, w), cb)
    qk = canonical_q2k(rng, 32)
    w = O.q2k_dequantize(qk, 32, 256)
    assert np.array_equal(gpu_quant(D.FMT_Q2K, w), qk)


def test_dequantize_bit_exact():
    rng = np.random.default_rng(10)
    w = (rng.standard_normal((48, 1024)) * 0.02).astype(np.float32)
    for fmt, quant, deq in ((D.FMT_CB2, O.cb2_quantize, O.cb2_dequantize), (D.FMT_Q2K, O.q2k_quantize, O.q2k_dequantize)):
        p = quant(w)
        got = gpu_dequant(fmt, p, 48, 1024)
        assert np.array_equal(got.view(np.uint32), deq(p, 48, 1024).view(np.uint32))


def test_dequantize_random_codes_bit_exact():
    """Arbitrary code bytes (every index, sign code and scale) with finite scales."""
    rng = np.random.default_rng(11)
    rows, cols = 16, 512
    n = rows * cols // 256
    codes = rng.integers(0, 256, n * 64, dtype=np.uint8)
    d = (np.abs(rng.standard_normal(n)) * 1e-3).astype(np.float16).view(np.uint16)
    cb = np.concatenate([codes, d.view(np.uint8)])
    assert np.array_equal(gpu_dequant(D.FMT_CB2, cb, rows, cols).view(np.uint32),
                          O.cb2_dequantize(cb, rows, cols).view(np.uint32))
    sub = rng.integers(0, 256, n * 16, dtype=np.uint8)
    sup = (np.abs(rng.standard_normal(2 * n)) * 1e-3).astype(np.float16).view(np.uint16)
    qk = np.concatenate([codes, sub, sup.view(np.uint8)])
    assert np.array_equal(gpu_dequant(D.FMT_Q2K, qk, rows, cols).view(np.uint32),
                          O.q2k_dequantize(qk, rows, cols).view(np.uint32))


def test_full_size_expert_quantize_byte_exact():
    """One routed expert at the DeepSeek V4 Flash shape (f 2048, d 4096)."""
    cfg = S.CONFIGS["decode1"]
    g, u, dn = S.gen_expert(cfg, 7)
    assert np.array_equal(gpu_quant(D.FMT_CB2, g), O.cb2_quantize(g))
    assert np.array_equal(gpu_quant(D.FMT_Q2K, dn), O.q2k_quantize(dn))


def test_empty_matrix_is_a_no_op():
    D.quantize(D.FMT_CB2, 0, 0, 256, 0)
    D.dequantize(D.FMT_Q2K, 0, 0, 512, 0)


# ------------------------------------------------------------------ MXFP4
def test_mx4_quantize_byte_exact():
    rng = np.random.default_rng(21)
    for rows, cols, scale in ((1, 256, 0.02), (37, 512, 0.02), (16, 4096, 1.0), (8, 768, 3e4)):
        w = (rng.standard_normal((rows, cols)) * scale).astype(np.float32)
        assert np.array_equal(gpu_quant(D.FMT_MXFP4, w), O.mx4_quantize(w)), (rows, cols, scale)


def test_mx4_quantize_edge_blocks_byte_exact():
    x = np.zeros((8, 256), dtype=np.float32)
    x[1, 17] = 0.5                                    # single spike
    x[2, :] = 1e-40                                   # subnormal inputs, scale clamps at 0
    x[3, 5], x[3, 6] = 3e38, -3e38                    # the largest scales
    x[4, :] = -0.01                                   # all negative
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.99, -0.25, -5.0, 0.1], dtype=np.float32)
    x[5, :12] = ties * 2.0 ** -6                      # every midpoint, and saturation
    x[6, :12] = ties * 2.0 ** 10
    x[7, ::3] = -1e-3                                 # negatives rounding to zero beside larger values
    x[7, 1::3] = 0.7
    assert np.array_equal(gpu_quant(D.FMT_MXFP4, x), O.mx4_quantize(x))


def test_mx4_dequantize_random_codes_bit_exact():
    """Every code byte with scale codes across the range (1 .. 252), and the
    quantizer's own output."""
    rng = np.random.default_rng(22)
    rows, cols = 16, 512
    n = rows * cols
    codes = rng.integers(0, 256, n // 2, dtype=np.uint8)
    codes[:256] = np.arange(256)
    scales = rng.integers(1, 253, n // 32).astype(np.uint8)
    p = np.concatenate([codes, scales])
    assert np.array_equal(gpu_dequant(D.FMT_MXFP4, p, rows, cols).view(np.uint32),
                          O.mx4_dequantize(p, rows, cols).view(np.uint32))
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    q = O.mx4_quantize(w)
    assert np.array_equal(gpu_dequant(D.FMT_MXFP4, q, rows, cols).view(np.uint32),
                          O.mx4_dequantize(q, rows, cols).view(np.uint32))


def test_mx4_full_size_expert_quantize_byte_exact():
    cfg = S.CONFIGS["decode1"]
    g, u, dn = S.gen_expert(cfg, 7)
    assert np.array_equal(gpu_quant(D.FMT_MXFP4, g), O.mx4_quantize(g))
    assert np.array_equal(gpu_quant(D.FMT_MXFP4, dn), O.mx4_quantize(dn))


# ------------------------------------------------------------------ Q4K
def test_q4k_quantize_byte_exact():
    rng = np.random.default_rng(31)
    for rows, cols, scale in ((1, 256, 0.02), (37, 512, 0.02), (16, 4096, 1.0), (8, 768, 3e4)):
        w = (rng.standard_normal((rows, cols)) * scale).astype(np.float32)
        assert np.array_equal(gpu_quant(D.FMT_Q4K, w), O.q4k_quantize(w)), (rows, cols, scale)


def test_q4k_quantize_edge_blocks_byte_exact():
    from tests.test_oracle_q4k import canonical_q4k
    x = np.zeros((6, 256), dtype=np.float32)
    x[1, 17] = 0.5                       # single spike
    x[2, :] = 1e-9                       # d underflows
    x[3, 5], x[3, 6] = 3e38, -3e38       # d clamps at 65504
    x[4, :] = -0.01                      # all negative
    x[5, ::2] = 0.03                     # exact ties
    x[5, 1::2] = -0.03
    assert np.array_equal(gpu_quant(D.FMT_Q4K, x), O.q4k_quantize(x))
    cq = canonical_q4k(np.random.default_rng(9), 16)
    w = O.q4k_dequantize(cq, 16, 256)
    assert np.array_equal(gpu_quant(D.FMT_Q4K, w), cq)


def test_q4k_dequantize_random_codes_bit_exact():
    rng = np.random.default_rng(32)
    rows, cols = 16, 512
    n = rows * cols // 256
    codes = rng.integers(0, 256, n * 128, dtype=np.uint8)
    scl = rng.integers(0, 256, n * 12, dtype=np.uint8)
    sup = (np.abs(rng.standard_normal(2 * n)) * 1e-3).astype(np.float16).view(np.uint16)
    p = np.concatenate([codes, scl, sup.view(np.uint8)])
    assert np.array_equal(gpu_dequant(D.FMT_Q4K, p, rows, cols).view(np.uint32),
                          O.q4k_dequantize(p, rows, cols).view(np.uint32))


def test_q4k_full_size_expert_quantize_byte_exact():
    cfg = S.CONFIGS["decode1"]
    g, u, dn = S.gen_expert(cfg, 7)
    assert np.array_equal(gpu_quant(D.FMT_Q4K, g), O.q4k_quantize(g))
    assert np.array_equal(gpu_quant(D.FMT_Q4K, dn), O.q4k_quantize(dn))
