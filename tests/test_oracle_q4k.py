"""Pins for the oracle's Q4K codec (CPU only): a hand-derived block layout
(tests/golden/q4k_layout.json), the decoder's closed form over every
(s, m, q), the quantizer's level choice against brute force, and the exact
round trip on canonical representable blocks."""
import json
import os

import numpy as np

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _le(words):
    return np.frombuffer(np.array(words, dtype=np.uint32).tobytes(), dtype=np.uint8)


def _word(elems: dict) -> int:
    """u32 of 8 codes: element 2p at bits 4p, element 2p + 1 at bits 16 + 4p."""
    u = 0
    for e, q in elems.items():
        p = e // 2
        u |= q << ((16 + 4 * p) if e % 2 else 4 * p)
    return u


def pack_block(codes: np.ndarray, s: np.ndarray, m: np.ndarray) -> tuple:
    """codes [256] (0..15), s/m [8] (0..63) -> (128 code bytes, 12 scale bytes)."""
    words = []
    for j in range(8):
        for k in range(4):
            words.append(_word({e: int(codes[32 * j + 8 * k + e]) for e in range(8)}))
    w0 = sum(int(s[j] & 15) << (4 * j) for j in range(8))
    w1 = sum(int(m[j] & 15) << (4 * j) for j in range(8))
    w2 = sum((int(s[j] >> 4) << (2 * j)) | (int(m[j] >> 4) << (16 + 2 * j)) for j in range(8))
    return _le(words), _le([w0, w1, w2])


def test_q4k_layout_golden():
    fx = json.load(open(os.path.join(GOLDEN, "q4k_layout.json")))
    codes = np.zeros(256, dtype=np.int64)
    for k, v in fx["codes"].items():
        codes[int(k)] = v
    s = np.zeros(8, dtype=np.int64)
    m = np.zeros(8, dtype=np.int64)
    s[0], m[0], s[1], m[1] = fx["scales"]["s0"], fx["scales"]["m0"], fx["scales"]["s1"], fx["scales"]["m1"]
    cb, sb = pack_block(codes, s, m)
    # the packer agrees with the words worked out by hand in the fixture
    assert sb.tobytes() == b"".join(bytes.fromhex(h)[::-1] for h in fx["scale_words_hex"])
    for off, h in fx["code_words_hex"].items():
        assert cb[int(off): int(off) + 4].tobytes() == bytes.fromhex(h)[::-1]
    sup = np.array([int(fx["d_bits"], 16), int(fx["dmin_bits"], 16)], dtype=np.uint16)
    w = O.q4k_dequantize(np.concatenate([cb, sb, sup.view(np.uint8)]), 1, 256)[0]
    for i, v in fx["values"].items():
        assert w[int(i)] == v, i


def test_q4k_dequant_closed_form_every_s_m_q():
    """d = 1, dmin = 0.5: every (s, m) pair on a sub-block, every q twice in
    it; the value is s * q - 0.5 * m (float32 steps in numpy)."""
    pairs = [(s, m) for s in range(64) for m in range(64)]
    rows = len(pairs) // 8
    cbs, sbs = [], []
    qv = np.tile(np.arange(16), 2)
    for r in range(rows):
        sm = pairs[8 * r: 8 * r + 8]
        s = np.array([a for a, _ in sm])
        m = np.array([b for _, b in sm])
        cb, sb = pack_block(np.tile(qv, 8), s, m)
        cbs.append(cb)
        sbs.append(sb)
    sup = np.tile(np.array([0x3C00, 0x3800], dtype=np.uint16), rows)
    packed = np.concatenate(cbs + sbs + [sup.view(np.uint8)])
    w = O.q4k_dequantize(packed, rows, 256)
    for r in range(rows):
        for j in range(8):
            s, m = pairs[8 * r + j]
            ref = np.float32(1.0) * np.float32(s) * qv.astype(np.float32) - np.float32(0.5) * np.float32(m)
            assert np.array_equal(w[r, 32 * j: 32 * j + 32], ref.astype(np.float32)), (s, m)


def test_q4k_level_choice_is_nearest():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((24, 512)) * 0.02).astype(np.float32)
    x[3] *= 1e3
    x[5, :32] = np.abs(x[5, :32])  # a sub-block without negatives (m = 0)
    p = O.q4k_quantize(x)
    codes, sc, sup = O.q4k_planes(p, 24, 512)
    w = O.q4k_dequantize(p, 24, 512)
    nb = 2
    for r in range(24):
        for b in range(nb):
            blk = r * nb + b
            d = np.float32(sup[2 * blk:2 * blk + 1].view(np.float16)[0])
            dmin = np.float32(sup[2 * blk + 1:2 * blk + 2].view(np.float16)[0])
            w0, w1, w2 = np.frombuffer(sc[12 * blk: 12 * blk + 12].tobytes(), dtype=np.uint32)
            for j in range(8):
                s = ((int(w0) >> (4 * j)) & 15) | (((int(w2) >> (2 * j)) & 3) << 4)
                m = ((int(w1) >> (4 * j)) & 15) | (((int(w2) >> (16 + 2 * j)) & 3) << 4)
                lv = (np.float32(d * np.float32(s)) * np.arange(16, dtype=np.float32)) - np.float32(dmin * np.float32(m))
                for i in range(32):
                    K = b * 256 + 32 * j + i
                    err = np.abs(lv - x[r, K])
                    assert w[r, K] == lv[int(np.argmin(err))], (r, K)


def canonical_q4k(rng, rows):
    """Exactly representable blocks with exact quantizer divisions: d, dmin
    normal and within 2^4 of each other, s_j >= 1 with one 63, one m_j = 63,
    every sub-block uses q = 0 and q = 15."""
    cbs, sbs, sups = [], [], []
    for _ in range(rows):
        e = int(rng.integers(-12, -8))
        em = e + int(rng.integers(-2, 3))
        sup = np.array([((e + 15) << 10) | int(rng.integers(0, 1024)), ((em + 15) << 10) | int(rng.integers(0, 1024))],
                       dtype=np.uint16)
        s = rng.integers(1, 64, 8)
        s[rng.integers(0, 8)] = 63
        m = rng.integers(0, 64, 8)
        m[rng.integers(0, 8)] = 63
        q = rng.integers(0, 16, 256)
        for j in range(8):
            pos = rng.permutation(32)[:2] + 32 * j
            q[pos[0]], q[pos[1]] = 0, 15
        cb, sb = pack_block(q, s, m)
        cbs.append(cb)
        sbs.append(sb)
        sups.append(sup)
    return np.concatenate(cbs + sbs + [np.concatenate(sups).view(np.uint8)])


def test_q4k_roundtrip_canonical_is_identity():
    rng = np.random.default_rng(6)
    packed = canonical_q4k(rng, 48)
    w = O.q4k_dequantize(packed, 48, 256)
    assert np.array_equal(O.q4k_quantize(w), packed)


def test_q4k_zero_block_and_quality():
    assert not O.q4k_quantize(np.zeros((2, 256), dtype=np.float32)).any()
    g = (np.random.default_rng(8).standard_normal((64, 512)) * 0.02).astype(np.float32)
    w = O.q4k_dequantize(O.q4k_quantize(g), 64, 512)
    rel = np.sqrt(((w - g) ** 2).mean() / (g ** 2).mean())
    assert rel < 0.1, rel
    assert ((w - g) ** 2).sum() < (g ** 2).sum()
