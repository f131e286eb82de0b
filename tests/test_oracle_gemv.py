"""Pins for the oracle's matrix-vector product.

* exact rational brute force on small matrices (Python Fractions from the
  logical codes and scales): the binary64 sequential sum must sit within
  (cols+1)*2^-53*S of the exact value;
* one-hot x returns a column of the dequantized matrix (rows != cols, so a
  transposed operand fails);
* linearity: scaling x by a power of two scales y exactly;
* the batched product equals per-token products;
* the row-range entry returns the matching slice.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def _exact_weights(fmt, L, rows, cols):
    """Exact dequantized weights as Fractions from the generator's logical values."""
    W = [[None] * cols for _ in range(rows)]
    if fmt == "q4_0":
        d, q = L["d"], L["q"]
        for i in range(rows):
            for j in range(cols):
                W[i][j] = (int(q[i, j]) - 8) * Fraction(float(d[i, j // 32]))
    elif fmt == "q8_0":
        d, q = L["d"], L["q"]
        for i in range(rows):
            for j in range(cols):
                W[i][j] = int(q[i, j]) * Fraction(float(d[i, j // 32]))
    elif fmt == "q4_k":
        d, dmin, sc, m, q = L["d"], L["dmin"], L["sc"], L["m"], L["q"]
        for i in range(rows):
            for j in range(cols):
                b, s = j // 256, (j % 256) // 32
                W[i][j] = (Fraction(float(d[i, b])) * int(sc[i, b, s]) * int(q[i, j])
                           - Fraction(float(dmin[i, b])) * int(m[i, b, s]))
    elif fmt == "q6_k":
        d, sc, q = L["d"], L["sc"], L["q"]
        for i in range(rows):
            for j in range(cols):
                W[i][j] = Fraction(float(d[i, j // 256])) * int(sc[i, j // 256, (j % 256) // 16]) * (int(q[i, j]) - 32)
    else:
        qq, s = L["q"], L["s"]
        for i in range(rows):
            for j in range(cols):
                W[i][j] = Fraction(float(s[i])) * int(qq[i, j])
    return W


@pytest.mark.parametrize("fmt,rows,cols", [("q4_0", 32, 32), ("q8_0", 32, 64),
                                           ("q4_k", 16, 256), ("q6_k", 16, 512), ("i8row", 32, 32)])
def test_brute_force_exact(fmt, rows, cols):
    rng = np.random.default_rng(11)
    t = synth.make_tensor(fmt, rows, cols, rng, keep_logical=True)
    x = rng.standard_normal((2, cols)).astype(np.float32)
    y, S = oracle.gemv(fmt, t.raw, x, rows, cols, row_scale=t.row_scale)
    W = _exact_weights(fmt, t.logical, rows, cols)
    w32 = oracle.dequant(fmt, t.raw, rows, cols, row_scale=t.row_scale)
    for tok in range(2):
        for i in range(rows):
            exact = sum(W[i][j] * Fraction(float(x[tok, j])) for j in range(cols))
            mag = sum(abs(W[i][j] * Fraction(float(x[tok, j]))) for j in range(cols))
            assert abs(Fraction(y[tok, i]) - exact) <= Fraction(cols + 1, 2 ** 53) * mag
            assert abs(Fraction(S[tok, i]) - mag) <= Fraction(cols + 1, 2 ** 53) * mag
    # the binary32 dequantized weight is the exact value rounded once
    for i in range(rows):
        for j in range(cols):
            assert w32[i, j] == np.float32(float(W[i][j])), (i, j)


@pytest.mark.parametrize("fmt,rows,cols", [("q4_0", 48, 96), ("q8_0", 40, 64),
                                           ("q4_k", 24, 512), ("q6_k", 24, 512), ("i8row", 40, 72)])
def test_one_hot_x_selects_column(fmt, rows, cols):
    rng = np.random.default_rng(12)
    t = synth.make_tensor(fmt, rows, cols, rng)
    w = oracle.dequant(fmt, t.raw, rows, cols, row_scale=t.row_scale).astype(np.float64)
    if fmt == "i8row":
        # s*q is exact in binary64 but rounded in the binary32 dequant
        w = t.row_scale.astype(np.float64)[:, None] * t.raw.astype(np.float64)
    for k in (0, 1, cols // 2 + 3, cols - 1):
        x = np.zeros(cols, np.float32)
        x[k] = 1.0
        y, S = oracle.gemv(fmt, t.raw, x, rows, cols, row_scale=t.row_scale)
        assert np.array_equal(y, w[:, k])
        assert np.array_equal(S, np.abs(w[:, k]))


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "q4_k", "q6_k", "i8row"])
def test_power_of_two_linearity_and_batching(fmt):
    rng = np.random.default_rng(13)
    rows, cols = 20, 512
    t = synth.make_tensor(fmt, rows, cols, rng)
    x = rng.standard_normal((3, cols)).astype(np.float32)
    y, S = oracle.gemv(fmt, t.raw, x, rows, cols, row_scale=t.row_scale)
    y8, S8 = oracle.gemv(fmt, t.raw, (x * np.float32(8.0)), rows, cols, row_scale=t.row_scale)
    assert np.array_equal(y8, 8.0 * y) and np.array_equal(S8, 8.0 * S)
    for tok in range(3):
        y1, S1 = oracle.gemv(fmt, t.raw, x[tok], rows, cols, row_scale=t.row_scale)
        assert np.array_equal(y1, y[tok]) and np.array_equal(S1, S[tok])
    # additivity within the binary64 bound
    x2 = rng.standard_normal(cols).astype(np.float32)
    xa = x[0].astype(np.float64) + x2.astype(np.float64)
    ya, _ = oracle.gemv_f64x(fmt, t.raw, xa, rows, cols, row_scale=t.row_scale)
    yb, Sb = oracle.gemv(fmt, t.raw, x2, rows, cols, row_scale=t.row_scale)
    assert np.all(np.abs(ya[0] - (y[0] + yb)) <= 4 * (cols + 1) * 2.0 ** -53 * (S[0] + Sb))


def test_row_range_is_a_slice():
    rng = np.random.default_rng(14)
    t = synth.make_tensor("q4_0", 64, 128, rng)
    x = rng.standard_normal((2, 128)).astype(np.float32)
    y, S = oracle.gemv("q4_0", t.raw, x, 64, 128)
    ys, Ss = oracle.gemv("q4_0", t.raw, x, 64, 128, row_begin=10, row_end=37)
    assert np.array_equal(ys, y[:, 10:37]) and np.array_equal(Ss, S[:, 10:37])


def test_f64x_matches_f32x_on_f32_values():
    rng = np.random.default_rng(15)
    t = synth.make_tensor("q8_0", 16, 64, rng)
    x = rng.standard_normal((2, 64)).astype(np.float32)
    y, S = oracle.gemv("q8_0", t.raw, x, 16, 64)
    y2, S2 = oracle.gemv_f64x("q8_0", t.raw, x.astype(np.float64), 16, 64)
    assert np.array_equal(y, y2) and np.array_equal(S, S2)
