"""Pins for the oracle's MXFP4 codec (CPU only): against the OCP MX value
tables and hand-worked blocks in tests/golden/mxfp4_spec.json, an exhaustive
closed form of the decoder, and a brute-force nearest-value search that
recomputes the shared exponent independently with numpy."""
import json
import math
import os

import numpy as np

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FX = json.load(open(os.path.join(GOLDEN, "mxfp4_spec.json")))
E2M1 = np.array(FX["e2m1_values"], dtype=np.float64)


def test_e2m1_all_codes_match_spec_table():
    for c in range(16):
        v = O.e2m1_value(c)
        assert v == E2M1[c]
        assert math.copysign(1.0, v) == math.copysign(1.0, E2M1[c])  # -0.0 for code 8


def test_e8m0_codes():
    vals = {"2^-127": 2.0 ** -127, "2^-126": 2.0 ** -126, "0.5": 0.5, "1": 1.0, "2": 2.0, "2^127": 2.0 ** 127}
    for code, want in FX["e8m0_cases"]:
        got = O.e8m0_value(code)
        if want == "NaN":
            assert math.isnan(got)
        else:
            assert got == vals[want], code


def test_mx4_sizes():
    assert O.mx4_bytes(2048, 4096) == 2048 * 4096 * 17 // 32 == 4456448
    assert O.mx4_bytes(4096, 2048) == 4456448


def test_mx4_golden_blocks():
    for b in FX["blocks"]:
        x = np.zeros((1, 256), dtype=np.float32)
        x[0, : len(b["x_head"])] = b["x_head"]
        p = O.mx4_quantize(x)
        codes, sc = O.mx4_planes(p, 1, 256)
        assert codes[:4].tobytes().hex() == b["code_bytes_head"], b["note"]
        assert not codes[4:16].any()
        assert int(sc[0]) == b["scale"]
        w = O.mx4_dequantize(p, 1, 256)[0]
        assert np.array_equal(w[: len(b["dequant_head"])], np.array(b["dequant_head"], dtype=np.float32))


def _pack(code_mat: np.ndarray, scale_row: np.ndarray) -> np.ndarray:
    """[rows, cols] nibble codes and [rows, cols/32] scale codes -> packed."""
    rows, cols = code_mat.shape
    lo, hi = code_mat[:, 0::2], code_mat[:, 1::2]
    codes = (lo | (hi << 4)).astype(np.uint8).ravel()
    return np.concatenate([codes, scale_row.astype(np.uint8).ravel()])


def test_mx4_dequant_closed_form_exhaustive():
    """Every code in every position, scale codes from the bottom to the top of
    the range: value = e2m1 * 2^(s - 127)."""
    rows, cols = 8, 256
    rng = np.random.default_rng(5)
    for scodes in ([0, 1, 100, 127, 130, 200, 252, 253], [90, 110, 120, 126, 128, 140, 150, 160]):
        cm = rng.integers(0, 16, (rows, cols))
        cm[:, :16] = np.arange(16)
        sm = np.repeat(np.array(scodes)[:, None], cols // 32, axis=1)
        sm[:, 1] = 127
        w = O.mx4_dequantize(_pack(cm, sm), rows, cols)
        ref = E2M1[cm] * np.exp2(np.repeat(sm, 32, axis=1).astype(np.float64) - 127)
        with np.errstate(over="ignore"):
            assert np.array_equal(w, ref.astype(np.float32))


def _brute_block(x: np.ndarray):
    """Shared exponent by the OCP rule with numpy's exact frexp, then every
    element's nearest of the 16 codes by exhaustive search (ties to the even
    code); codes of zero magnitude are stored as +0."""
    amax = float(np.max(np.abs(x.astype(np.float64))))
    if amax == 0.0:
        return 0, np.zeros(32, dtype=np.int64)
    _, ex = np.frexp(amax)
    s = min(max(int(ex) - 1 - 2 + 127, 0), 254)
    r = x.astype(np.float64) / 2.0 ** (s - 127)
    codes = np.zeros(32, dtype=np.int64)
    for i in range(32):
        err = np.abs(E2M1[:8] - abs(r[i]))
        best = [c for c in range(8) if err[c] == err.min()]
        c = min(best, key=lambda c: (c & 1, c))  # even code on a tie
        codes[i] = c | (8 if (x[i] < 0 and c != 0) else 0)
    return s, codes


def test_mx4_quantizer_matches_brute_force():
    rng = np.random.default_rng(11)
    blocks = [rng.standard_normal(32) * 0.02, rng.standard_normal(32), rng.standard_normal(32) * 1e4,
              rng.standard_normal(32) * 1e-30, np.exp(rng.uniform(-20, 20, 32)) * rng.choice([-1, 1], 32)]
    for _ in range(40):
        blocks.append(rng.standard_normal(32) * 10.0 ** rng.uniform(-6, 6))
    # exact ties and saturation at every binade
    for s in (-8, 0, 5):
        blocks.append(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.99, -0.25, -5.0] + [0.1] * 21) * 2.0 ** s)
    x = np.array(blocks, dtype=np.float32).reshape(-1, 32)
    rows = len(x) // 8 * 8
    X = x[:rows].reshape(rows // 8, 256)
    p = O.mx4_quantize(X)
    codes, sc = O.mx4_planes(p, X.shape[0], 256)
    nib = np.stack([codes & 15, codes >> 4], axis=1).reshape(-1)  # element order
    for b in range(rows):
        s, c = _brute_block(x[b])
        assert int(sc[b]) == s, b
        assert np.array_equal(nib[32 * b: 32 * b + 32], c), b


def test_mx4_roundtrip_on_representable_blocks():
    """Blocks whose largest element is 4 or 6 times 2^k, all elements on the
    E2M1 grid times 2^k: the rule recovers 2^k and the codes, so
    dequantize(quantize(w)) == w bit for bit."""
    rng = np.random.default_rng(17)
    rows, cols = 16, 256
    cm = rng.integers(0, 16, (rows, cols))
    cm[:, ::32] = rng.choice([6, 7, 14, 15], (rows, cols // 32))  # a 4 or 6 in every block
    sm = rng.integers(100, 150, (rows, cols // 32))
    w = O.mx4_dequantize(_pack(cm, sm), rows, cols)
    p2 = O.mx4_quantize(w)
    assert np.array_equal(O.mx4_dequantize(p2, rows, cols), w)
    codes2, sc2 = O.mx4_planes(p2, rows, cols)
    assert np.array_equal(sc2.reshape(rows, -1), sm)


def test_mx4_zero_block_and_quality():
    x = np.zeros((2, 256), dtype=np.float32)
    assert not O.mx4_quantize(x).any()
    g = np.random.default_rng(3).standard_normal((64, 512)).astype(np.float32) * 0.02
    w = O.mx4_dequantize(O.mx4_quantize(g), 64, 512)
    rel = np.sqrt(((w - g) ** 2).mean() / (g ** 2).mean())
    assert rel < 0.2, rel  # 4-bit elements with a power-of-two scale per 32
