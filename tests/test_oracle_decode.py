"""Pins for the oracle's block decoders, independent of the oracle itself.

Each check comes from a definition on the pages or from mathematics: the IEEE
binary16 definition (checked exhaustively against numpy's conversion), closed
forms of hand-built blocks (zero scale, neutral code, one-hot codes) and the
hand-worked fixtures in tests/golden/.  Hand-built blocks are assembled byte
by byte here, not with the generator's packers.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests import _golden as G


# ---------------------------------------------------------------- f16 ------
def test_f16_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # the sign of zero survives
    assert math.copysign(1.0, oracle.f16_to_f64(0x8000)) == -1.0


def test_f16_golden():
    g = G.load("f16_values.json")
    for c in g["cases"]:
        v = oracle.f16_to_f64(int(c["bits"], 16))
        want = G.num(c["value"])
        if math.isnan(want):
            assert math.isnan(v), c
        else:
            assert v == want and math.copysign(1, v) == math.copysign(1, want), c


# ---------------------------------------------------------------- Q8_0 -----
def _q8_block(d_bits, codes):
    blk = np.zeros(34, dtype=np.uint8)
    blk[0] = d_bits & 0xFF
    blk[1] = d_bits >> 8
    blk[2:] = np.asarray(codes, dtype=np.int64) & 0xFF
    return blk


def test_q8_0_exhaustive_byte_and_position():
    # every byte value at every position, scale 1.0: the weight is the signed
    # byte and it sits in its own column
    rows = []
    for v in range(256):
        for pos in range(32):
            codes = np.zeros(32, dtype=np.int64)
            codes[pos] = v
            rows.append(_q8_block(0x3C00, codes))
    raw = np.stack(rows)
    w = oracle.dequant("q8_0", raw, len(rows), 32)
    k = 0
    for v in range(256):
        signed = v - 256 if v >= 128 else v
        for pos in range(32):
            expect = np.zeros(32, dtype=np.float32)
            expect[pos] = signed
            assert np.array_equal(w[k], expect), (v, pos)
            k += 1


def test_q8_0_zero_scale_gives_zero():
    rng = np.random.default_rng(1)
    raw = np.stack([_q8_block(0x0000, rng.integers(-128, 128, 32)) for _ in range(8)])
    w = oracle.dequant("q8_0", raw, 8, 32)
    assert np.all(w == 0)


def test_q8_0_golden_block():
    g = G.load("q8_0_block.json")
    raw = G.hexbytes(g["block_hex"]).reshape(1, 34)
    w = oracle.dequant("q8_0", raw, 1, 32)[0]
    expect = np.zeros(32)
    for col, v in g["expected_nonzero"].items():
        expect[int(col)] = G.num(v)
    assert np.array_equal(w, expect.astype(np.float32))
    y, S = oracle.gemv("q8_0", raw, np.ones(32, np.float32), 1, 32)
    assert y[0] == G.num(g["y_ones"])


# ---------------------------------------------------------------- Q4_0 -----
def _q4_0_block(d_bits, codes32):
    """codes32[c] is the code of column c (0..15)."""
    c = np.asarray(codes32, dtype=np.int64)
    blk = np.zeros(18, dtype=np.uint8)
    blk[0] = d_bits & 0xFF
    blk[1] = d_bits >> 8
    for l in range(16):
        blk[2 + l] = (c[l] & 0xF) | ((c[16 + l] & 0xF) << 4)
    return blk


def test_q4_0_zero_scale_gives_zero():
    rng = np.random.default_rng(2)
    raw = np.stack([_q4_0_block(0, rng.integers(0, 16, 32)) for _ in range(4)])
    w = oracle.dequant("q4_0", raw, 4, 32)
    assert np.all(w == 0)
    y, S = oracle.gemv("q4_0", raw, rng.standard_normal(32).astype(np.float32), 4, 32)
    assert np.all(y == 0) and np.all(S == 0)


def test_q4_0_code_eight_is_zero():
    raw = np.stack([_q4_0_block(b, [8] * 32) for b in (0x3C00, 0xC000, 0x7BFF, 0x0001)])
    w = oracle.dequant("q4_0", raw, 4, 32)
    assert np.all(w == 0)


def test_q4_0_constant_codes_closed_form():
    # every code = q: y = (q-8) * d * sum(x), evaluated exactly with Fractions
    from fractions import Fraction
    rng = np.random.default_rng(3)
    x = rng.standard_normal(32).astype(np.float32)
    sx = sum(Fraction(float(v)) for v in x)
    for q in range(16):
        for d_bits in (0x3C00, 0x2E66, 0xB555):
            raw = _q4_0_block(d_bits, [q] * 32).reshape(1, 18)
            d = Fraction(float(np.array([d_bits], np.uint16).view(np.float16)[0]))
            y, S = oracle.gemv("q4_0", raw, x, 1, 32)
            exact = (q - 8) * d * sx
            assert abs(Fraction(y[0]) - exact) <= Fraction(33, 2 ** 53) * Fraction(S[0]) + Fraction(1, 10 ** 300)


def test_q4_0_one_hot_code_locates_column():
    # 16 values x 32 positions; neutral code 8 elsewhere
    rows = []
    for v in range(16):
        for pos in range(32):
            c = [8] * 32
            c[pos] = v
            rows.append(_q4_0_block(0x3800, c))     # d = 0.5
    w = oracle.dequant("q4_0", np.stack(rows), len(rows), 32)
    k = 0
    for v in range(16):
        for pos in range(32):
            expect = np.zeros(32, np.float32)
            expect[pos] = (v - 8) * 0.5
            assert np.array_equal(w[k], expect), (v, pos)
            k += 1


def test_q4_0_golden_block():
    g = G.load("q4_0_block.json")
    raw = G.hexbytes(g["block_hex"]).reshape(1, 18)
    w = oracle.dequant("q4_0", raw, 1, 32)[0]
    expect = np.zeros(32, np.float32)
    for col, v in g["expected_nonzero"].items():
        expect[int(col)] = G.num(v)
    assert np.array_equal(w, expect)
    y, _ = oracle.gemv("q4_0", raw, np.ones(32, np.float32), 1, 32)
    assert y[0] == G.num(g["y_ones"])


# ---------------------------------------------------------------- Q4_K -----
def test_q4_k_scale_min_golden():
    g = G.load("q4_k_block.json")
    sc12 = G.hexbytes(g["scales_hex"])
    for j, (sc, m, _) in enumerate(g["scale_min"]):
        assert oracle.q4k_scale_min(j, sc12) == (sc, m), j


def test_q4_k_scale_min_bijection_exhaustive_per_position():
    # For each sub-block position, every (sc, m) pair in 64x64, embedded in
    # random surrounding bytes, is recovered: the 12-byte field carries eight
    # independent six-bit pairs.  The field is assembled bit by bit here.
    rng = np.random.default_rng(4)
    for j in range(8):
        for sc in range(64):
            for m in range(0, 64, 7):
                pairs_sc = rng.integers(0, 64, 8)
                pairs_m = rng.integers(0, 64, 8)
                pairs_sc[j], pairs_m[j] = sc, m
                f = np.zeros(12, np.int64)
                for i in range(4):
                    f[i] = pairs_sc[i] | ((pairs_sc[i + 4] >> 4) << 6)
                    f[i + 4] = pairs_m[i] | ((pairs_m[i + 4] >> 4) << 6)
                    f[i + 8] = (pairs_sc[i + 4] & 15) | ((pairs_m[i + 4] & 15) << 4)
                got = [oracle.q4k_scale_min(i, f.astype(np.uint8)) for i in range(8)]
                assert got == list(zip(pairs_sc.tolist(), pairs_m.tolist())), (j, sc, m)


def test_q4_k_scale_min_every_byte_string_is_some_pairs():
    # the map is onto six-bit pairs and injective: random strings round-trip
    rng = np.random.default_rng(5)
    for _ in range(2000):
        f = rng.integers(0, 256, 12).astype(np.uint8)
        pairs = [oracle.q4k_scale_min(i, f) for i in range(8)]
        assert all(0 <= a < 64 and 0 <= b < 64 for a, b in pairs)
        g = np.zeros(12, np.int64)
        for i in range(4):
            g[i] = pairs[i][0] | ((pairs[i + 4][0] >> 4) << 6)
            g[i + 4] = pairs[i][1] | ((pairs[i + 4][1] >> 4) << 6)
            g[i + 8] = (pairs[i + 4][0] & 15) | ((pairs[i + 4][1] & 15) << 4)
        assert np.array_equal(g.astype(np.uint8), f)


def _q4_k_block(d_bits, dmin_bits, scales12, codes256):
    c = np.asarray(codes256, np.int64).reshape(8, 32)
    blk = np.zeros(144, np.uint8)
    blk[0], blk[1] = d_bits & 0xFF, d_bits >> 8
    blk[2], blk[3] = dmin_bits & 0xFF, dmin_bits >> 8
    blk[4:16] = scales12
    for ch in range(4):
        for l in range(32):
            blk[16 + 32 * ch + l] = (c[2 * ch, l] & 15) | ((c[2 * ch + 1, l] & 15) << 4)
    return blk


def test_q4_k_golden_block():
    g = G.load("q4_k_block.json")
    b = g["block"]
    blk = np.zeros(144, np.uint8)
    blk[0:2] = G.hexbytes(b["d_hex"])
    blk[2:4] = G.hexbytes(b["dmin_hex"])
    blk[4:16] = G.hexbytes(g["scales_hex"])
    for off, hx in b["qs_set"].items():
        blk[16 + int(off)] = int(hx, 16)
    w = oracle.dequant("q4_k", blk.reshape(1, 144), 1, 256)[0]
    for col, v in b["expected"].items():
        assert w[int(col)] == G.num(v), col
    y, _ = oracle.gemv("q4_k", blk.reshape(1, 144), np.ones(256, np.float32), 1, 256)
    assert y[0] == G.num(b["y_ones"])


def test_q4_k_closed_forms():
    rng = np.random.default_rng(6)
    sc = rng.integers(0, 64, 8)
    m = rng.integers(0, 64, 8)
    f = np.zeros(12, np.int64)
    for i in range(4):
        f[i] = sc[i] | ((sc[i + 4] >> 4) << 6)
        f[i + 4] = m[i] | ((m[i + 4] >> 4) << 6)
        f[i + 8] = (sc[i + 4] & 15) | ((m[i + 4] & 15) << 4)
    f = f.astype(np.uint8)
    zero12 = np.zeros(12, np.uint8)
    codes = rng.integers(0, 16, 256)
    d, dmin = 0x3C00, 0x3800            # 1.0, 0.5
    # sc = m = 0: every weight is zero
    w = oracle.dequant("q4_k", _q4_k_block(d, dmin, zero12, codes).reshape(1, 144), 1, 256)[0]
    assert np.all(w == 0)
    # q = 0: w = -dmin*m (the minimum is subtracted)
    w = oracle.dequant("q4_k", _q4_k_block(d, dmin, f, np.zeros(256)).reshape(1, 144), 1, 256)[0]
    assert np.array_equal(w, np.repeat(-0.5 * m, 32).astype(np.float32))
    # dmin = 0: w = d*sc*q
    w = oracle.dequant("q4_k", _q4_k_block(d, 0, f, codes).reshape(1, 144), 1, 256)[0]
    assert np.array_equal(w, (np.repeat(sc, 32) * codes).astype(np.float32))
    # d = 0: w = -dmin*m whatever the codes
    w = oracle.dequant("q4_k", _q4_k_block(0, dmin, f, codes).reshape(1, 144), 1, 256)[0]
    assert np.array_equal(w, np.repeat(-0.5 * m, 32).astype(np.float32))


def test_q4_k_one_hot_code_locates_column():
    # scales all 1, mins 0, d = 1: one code set to 5 at each position in turn
    ones = np.zeros(12, np.int64)
    for i in range(4):
        ones[i] = 1
        ones[i + 8] = 1
    ones = ones.astype(np.uint8)
    rows = []
    for pos in range(256):
        c = np.zeros(256, np.int64)
        c[pos] = 5
        rows.append(_q4_k_block(0x3C00, 0, ones, c))
    w = oracle.dequant("q4_k", np.stack(rows), 256, 256)
    assert np.array_equal(w, 5 * np.eye(256, dtype=np.float32))


# ---------------------------------------------------------------- Q6_K -----
def _q6_k_block(d_bits, scales16, codes256):
    """One 210-byte super-block assembled byte by byte from 256 six-bit codes
    (column c = 128h + 32j + l: low bits to ql[64h + 32(j mod 2) + l], nibble
    j >= 2; top bits to bits 2j of qh[32h + l])."""
    c = np.asarray(codes256, np.int64)
    blk = np.zeros(210, np.int64)
    for col in range(256):
        h, j, l = col // 128, (col % 128) // 32, col % 32
        blk[64 * h + 32 * (j % 2) + l] |= (c[col] & 15) << (4 if j >= 2 else 0)
        blk[128 + 32 * h + l] |= (c[col] >> 4) << (2 * j)
    blk[192:208] = np.asarray(scales16, np.int64) & 0xFF
    blk[208], blk[209] = d_bits & 0xFF, d_bits >> 8
    return blk.astype(np.uint8)


def test_q6_k_golden_block():
    g = G.load("q6_k_block.json")
    blk = np.zeros(210, np.uint8)
    blk[192:208] = G.hexbytes(g["scales_hex"])
    blk[208:210] = G.hexbytes(g["d_hex"])
    for off, hx in g["bytes_set"].items():
        blk[int(off)] = int(hx, 16)
    w = oracle.dequant("q6_k", blk.reshape(1, 210), 1, 256)[0]
    for col, v in g["expected"].items():
        assert w[int(col)] == G.num(v), col
    y, _ = oracle.gemv("q6_k", blk.reshape(1, 210), np.ones(256, np.float32), 1, 256)
    assert y[0] == G.num(g["y_ones"])


def test_q6_k_bits_per_weight_is_the_pages_figure():
    # 128 + 64 code bytes, 16 scale bytes and a 2-byte f16 per 256 weights:
    # 6.5625 bits per weight, the "about 6.6" of the pages
    per, nbytes = synth.FMT_BLOCK["q6_k"]
    assert (per, nbytes) == (256, 210) and abs(8 * nbytes / per - 6.6) < 0.05
    # the decoder's super-block and row strides are 210 bytes: a row of three
    # blocks with d = 1, 2, 4 and every code 33 (w = d * sc)
    ones = np.ones(16, np.int64)
    rows = [np.concatenate([_q6_k_block(b, ones, np.full(256, 33)) for b in ds])
            for ds in ((0x3C00, 0x4000, 0x4400), (0x4400, 0x3800, 0x3C00))]
    w = oracle.dequant("q6_k", np.stack(rows), 2, 768)
    assert np.array_equal(w, np.repeat(np.float32([[1, 2, 4], [4, 0.5, 1]]), 256, axis=1))


def test_q6_k_closed_forms():
    rng = np.random.default_rng(16)
    codes = rng.integers(0, 64, 256)
    sc = rng.integers(-128, 128, 16)
    # d = 0, scales 0, or every code at the offset 32: every weight is zero
    for d_bits, s16, c in ((0, sc, codes), (0x3C00, np.zeros(16, np.int64), codes), (0x3C00, sc, np.full(256, 32))):
        w = oracle.dequant("q6_k", _q6_k_block(d_bits, s16, c).reshape(1, 210), 1, 256)[0]
        assert np.all(w == 0)
    # every code value at every position (scale 1, d = 1): w = q - 32
    for k in range(4):
        c = (np.arange(256) * 5 + 17 * k) % 64
        w = oracle.dequant("q6_k", _q6_k_block(0x3C00, np.ones(16, np.int64), c).reshape(1, 210), 1, 256)[0]
        assert np.array_equal(w, (c - 32).astype(np.float32))


def test_q6_k_scales_are_signed_bytes():
    # all 256 scale bytes over 16 blocks, code 33, d = 0.25: w = sc / 4 with
    # sc the two's-complement value of the byte
    rows = [_q6_k_block(0x3400, np.arange(16 * b, 16 * b + 16), np.full(256, 33)) for b in range(16)]
    w = oracle.dequant("q6_k", np.stack(rows), 16, 256)
    sc = np.arange(256).astype(np.uint8).view(np.int8).astype(np.float32)
    assert np.array_equal(w, 0.25 * np.repeat(sc.reshape(16, 16), 16, axis=1))


def test_q6_k_single_bit_locates_column():
    # every code at 32 (ql 0x00, qh 0xAA): all weights zero; one flipped bit
    # moves exactly one column, the one the layout names
    base = np.zeros(210, np.uint8)
    base[128:192] = 0xAA
    base[192:208] = 1
    base[208:210] = (0x00, 0x3C)
    rows, want = [], []
    for i in range(192):
        for bit in range(8):
            b = base.copy()
            b[i] ^= 1 << bit
            rows.append(b)
            if i < 128:
                col = 128 * (i // 64) + i % 64 + (64 if bit >= 4 else 0)
                val = 2 ** (bit % 4)
            else:
                k = i - 128
                col = 128 * (k // 32) + 32 * (bit // 2) + k % 32
                val = 16 if bit % 2 == 0 else -32
            want.append((col, val))
    w = oracle.dequant("q6_k", np.stack(rows), len(rows), 256)
    for r, (col, val) in enumerate(want):
        nz = np.flatnonzero(w[r])
        assert list(nz) == [col] and w[r, col] == val, (r // 8, r % 8)


# ---------------------------------------------------------------- I8ROW ----
def test_i8row_golden():
    g = G.load("i8row_row.json")
    q = np.array(g["codes"], np.int8).reshape(1, 4)
    s = np.array([g["row_scale"]], np.float32)
    w = oracle.dequant("i8row", q, 1, 4, row_scale=s)[0]
    assert np.array_equal(w, np.array([G.num(e) for e in g["expected"]], np.float32))
    y, _ = oracle.gemv("i8row", q, np.ones(4, np.float32), 1, 4, row_scale=s)
    assert y[0] == G.num(g["y_ones"])


def test_i8row_unit_scale_one_hot_gives_integer_column():
    rng = np.random.default_rng(7)
    q = rng.integers(-127, 128, (24, 40)).astype(np.int8)
    s = np.ones(24, np.float32)
    for k in (0, 17, 39):
        x = np.zeros(40, np.float32)
        x[k] = 1
        y, _ = oracle.gemv("i8row", q, x, 24, 40, row_scale=s)
        assert np.array_equal(y, q[:, k].astype(np.float64))


def test_i8row_power_of_two_scale_ones_gives_scaled_row_sum():
    rng = np.random.default_rng(8)
    q = rng.integers(-127, 128, (16, 64)).astype(np.int8)
    for k in (-12, 0, 5):
        s = np.full(16, 2.0 ** k, np.float32)
        y, _ = oracle.gemv("i8row", q, np.ones(64, np.float32), 16, 64, row_scale=s)
        assert np.array_equal(y, (2.0 ** k) * q.astype(np.int64).sum(1))


def test_i8row_dequant_rounds_once():
    # s*q is formed exactly and rounded once to binary32
    s = np.array([0.1, 1e-3, 3.0e-4], np.float32)
    q = np.array([[127, -127, 3], [1, 2, -77], [100, -1, 55]], np.int8)
    w = oracle.dequant("i8row", q, 3, 3, row_scale=s)
    expect = (s.astype(np.float64)[:, None] * q.astype(np.float64)).astype(np.float32)
    assert np.array_equal(w, expect)


@pytest.mark.parametrize("fmt,cols", [("q4_0", 33), ("q8_0", 48), ("q4_k", 300), ("q6_k", 320)])
def test_shape_refusals(fmt, cols):
    with pytest.raises(ValueError):
        oracle.dequant(fmt, np.zeros(4096, np.uint8), 1, cols)
