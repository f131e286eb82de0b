"""Pins for the oracle's Q8_0 activation path (the Go "llm" package's
ExactGGML mode: activations quantised to Q8_0 before each quantised product).

* binary32 -> binary16 rounding (nearest even) against numpy's conversion on
  every binary16 value, every midpoint between neighbours and points beside
  them, subnormals, the overflow edge and random values over all binades;
* the quantizer on hand-worked blocks (ties, negative maxima, zero blocks, a
  non-power-of-two scale) and on invariants (the largest magnitude maps to
  +-127, every element within half a step of its code);
* the product: on activations already on the Q8_0 grid it equals the plain
  product exactly; otherwise it equals an exact rational evaluation from the
  quantized codes, and stays within the quantization error of the plain one.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import _golden as G


def test_f32_to_f16_matches_numpy():
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)      # every finite positive binary16
    v = h.view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2                                      # exact ties (representable in binary32)
    pts = np.concatenate([v, mids, 65504.0 + np.array([0, 8, 15.99, 16, 16.01, 100])])
    pts32 = pts.astype(np.float32)
    beside = np.concatenate([np.nextafter(pts32, np.float32(np.inf)), np.nextafter(pts32, np.float32(0))])
    rng = np.random.default_rng(30)
    rnd = (rng.standard_normal(20000) * 2.0 ** rng.integers(-30, 20, 20000)).astype(np.float32)
    allv = np.concatenate([pts32, beside, rnd, np.float32([0.0, np.inf, 1e-30, 3e38])])
    allv = np.concatenate([allv, -allv])
    with np.errstate(over="ignore"):
        want = allv.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16(f) for f in allv], dtype=np.uint16)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(allv[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_quantize_golden_blocks():
    g = G.load("q8_0_activation.json")
    for blk in g["blocks"]:
        x = np.zeros(32, np.float32)
        for k, v in blk["x"].items():
            x[int(k)] = v
        d, q = oracle.quantize_q8_0(x)
        assert d[0] == int(blk["d_bits"], 16), blk["working"]
        for k, v in blk["q"].items():
            assert int(q[int(k)]) == v, (k, blk["working"])
        assert np.count_nonzero(q) == sum(1 for v in blk["q"].values() if v), blk["working"]


def test_quantize_exact_grid_and_invariants():
    rng = np.random.default_rng(31)
    # x = k * 2^e with max |k| = 127: d = 2^e exactly and the codes are k
    for e in (-20, -3, 0, 5):
        k = rng.integers(-127, 128, (4, 64))
        k[:, 0], k[:, 32] = 127, -127
        x = (k * 2.0 ** e).astype(np.float32)
        d, q = oracle.quantize_q8_0(x)
        assert np.array_equal(q, k) and np.all(d == np.float16(2.0 ** e).view(np.uint16))
    # random blocks: the largest magnitude maps to +-127 with its sign, every
    # element lies within half a step (binary32 step) of its code
    x = (rng.standard_normal((8, 256)) * 3).astype(np.float32)
    d, q = oracle.quantize_q8_0(x)
    xb, qb = x.reshape(-1, 32).astype(np.float64), q.reshape(-1, 32).astype(np.float64)
    amax = np.abs(xb).max(1)
    step = (amax.astype(np.float32) / np.float32(127)).astype(np.float64)
    i = np.abs(xb).argmax(1)
    assert np.array_equal(qb[np.arange(len(i)), i], 127 * np.sign(xb[np.arange(len(i)), i]))
    assert np.all(np.abs(xb - step[:, None] * qb) <= step[:, None] * (0.5 + 1e-5))
    assert np.array_equal(d.reshape(-1), step.astype(np.float32).astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_gemv_q8act_on_grid_equals_plain(fmt):
    # activations already on the Q8_0 grid (power-of-two steps, max code 127):
    # the representation is x itself, so the product is the plain one, exactly
    rng = np.random.default_rng(32)
    rows, cols = 40, 512
    t = synth.make_tensor(fmt, rows, cols, rng)
    k = rng.integers(-127, 128, (2, cols))
    k[:, ::32] = 127
    x = (k * 2.0 ** -6).astype(np.float32)
    y8, S8 = oracle.gemv_q8act(fmt, t.raw, x, rows, cols)
    y, S = oracle.gemv(fmt, t.raw, x, rows, cols)
    assert np.array_equal(y8, y) and np.array_equal(S8, S)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_gemv_q8act_brute_force_and_quantization_error(fmt):
    rng = np.random.default_rng(33)
    rows, cols = 12, 128
    t = synth.make_tensor(fmt, rows, cols, rng, keep_logical=True)
    x = rng.standard_normal(cols).astype(np.float32)
    y8, S8 = oracle.gemv_q8act(fmt, t.raw, x, rows, cols)
    d, q = oracle.quantize_q8_0(x)
    L = t.logical
    for i in range(rows):
        exact = Fraction(0)
        for b in range(cols // 32):
            dw = Fraction(float(L["d"][i, b]))
            dx = Fraction(float(np.uint16(d[b]).view(np.float16)))
            codes = [(int(L["q"][i, 32 * b + l]) - (8 if fmt == "q4_0" else 0)) * int(q[32 * b + l])
                     for l in range(32)]
            exact += dw * dx * sum(codes)
        assert abs(Fraction(y8[i]) - exact) <= Fraction(cols + 1, 2 ** 53) * Fraction(S8[i])
    # against the plain product: within sum_j |w_ij| |x_j - xq_j|
    y, _ = oracle.gemv(fmt, t.raw, x, rows, cols)
    w = oracle.dequant(fmt, t.raw, rows, cols).astype(np.float64)
    xq = np.repeat(np.uint16(d).view(np.float16).astype(np.float64), 32) * q
    gap = np.abs(w) @ np.abs(x.astype(np.float64) - xq)
    assert np.all(np.abs(y8 - y) <= gap * (1 + 1e-12) + 1e-300)
    assert np.any(y8 != y)


def test_gemv_q8act_refuses_other_formats():
    with pytest.raises(ValueError):
        oracle.gemv_q8act("q4_k", np.zeros(144, np.uint8), np.zeros(256, np.float32), 1, 256)
    with pytest.raises(ValueError):
        oracle.quantize_q8_0(np.zeros(40, np.float32))
