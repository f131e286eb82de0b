"""Pins for the oracle's RMSNorm and the FFN block of the residual stream.

RMSNorm (llmoxide blog, section 4 "Keeping the numbers in range"; dasLLAMA-00's
rmsnorm): scale = 1/sqrt(mean(x^2) + eps), out_j = x_j * scale * gamma_j.
The block (same blog, section 7 "The block, and the residual stream"):
out = x + Wd (silu(Wg xn) * (Wu xn)), xn = rmsnorm(x) * gamma.

* hand-worked values (tests/golden/rmsnorm_values.json), including a case that
  separates eps inside the root from eps outside and the mean from the sum;
* closed form for a constant row, c*gamma_j/sqrt(c^2 + eps);
* with eps = 0: unit root-mean-square output, and invariance under scaling x
  by a power of two (bit-exact);
* the block with identity-pattern Q8_0 matrices reduces to
  out = x + silu(xn) * 2 xn (gate = xn, up = 2 xn, down = identity);
* zero down scales or a zero gain leave out == x exactly (the residual).
"""
import numpy as np
from scipy.special import expit

import oracle
import synth
from tests import _golden as G


def test_rmsnorm_golden():
    for c in G.load("rmsnorm_values.json")["cases"]:
        x = np.array(c["x"], np.float32)
        out, sc = oracle.rmsnorm(x, np.array(c["gamma"], np.float32), c["eps"])
        assert abs(sc - c["scale"]) <= 4e-16 * abs(c["scale"]), c["working"]
        want = np.array(c["out"])
        assert np.all(np.abs(out - want) <= 4e-16 * np.maximum(np.abs(want), 1e-300)), c["working"]


def test_rmsnorm_constant_row_closed_form():
    n = 96
    gamma = np.random.default_rng(31).uniform(-2, 2, n).astype(np.float32)
    for c, eps in ((0.5, 1e-5), (-3.0, 1e-6), (7.25, 0.0), (1e-3, 1e-5)):
        out, _ = oracle.rmsnorm(np.full(n, c, np.float32), gamma, eps)
        c64 = float(np.float32(c))
        want = c64 * gamma.astype(np.float64) / np.sqrt(c64 * c64 + eps)
        assert np.all(np.abs(out - want) <= 1e-15 * np.abs(want) + 1e-300)


def test_rmsnorm_unit_rms_and_power_of_two_invariance():
    rng = np.random.default_rng(32)
    x = rng.standard_normal((4, 288)).astype(np.float32)
    ones = np.ones(288, np.float32)
    out, _ = oracle.rmsnorm(x, ones, 0.0)
    assert np.all(np.abs(np.mean(out * out, axis=1) - 1.0) <= 1e-14)
    for k in (-6, 3, 11):
        out_k, _ = oracle.rmsnorm(x * np.float32(2.0 ** k), ones, 0.0)
        assert np.array_equal(out_k, out)


def _identity_q8(n, d_bits=0x3C00):
    q = np.zeros((n, n), np.int8)
    q[np.arange(n), np.arange(n)] = 1
    d = np.full((n, n // 32), np.uint16(d_bits)).view(np.float16)
    return synth.pack_q8_0(d, q)


def test_block_identity_closed_form():
    # gate = xn, up = 2 xn (scale 2), down = identity: out = x + silu(xn) * 2 xn
    n = 64
    rng = np.random.default_rng(33)
    x = rng.standard_normal((3, n)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, n).astype(np.float32)
    eps = 1e-5
    r = oracle.ffn_block("q8_0", _identity_q8(n), _identity_q8(n, 0x4000), _identity_q8(n), gamma, eps, x, n, n)
    xn, _ = oracle.rmsnorm(x, gamma, eps)
    assert np.array_equal(r["xn"], xn)
    h = xn * expit(xn) * 2 * xn
    assert np.all(np.abs(r["h"] - h) <= 1e-15 * np.maximum(1, np.abs(h)))
    want = x.astype(np.float64) + h
    assert np.all(np.abs(r["out"] - want) <= 1e-15 * np.maximum(1, np.abs(want)))


def test_block_zero_down_or_zero_gain_is_the_residual():
    d_model, ffn = 64, 96
    rng = np.random.default_rng(34)
    x = rng.standard_normal((2, d_model)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, d_model).astype(np.float32)
    tg = synth.make_tensor("q4_0", ffn, d_model, rng)
    tu = synth.make_tensor("q4_0", ffn, d_model, rng)
    dd, qd = synth.draw_q4_0(rng, d_model, ffn)
    wd0 = synth.pack_q4_0(np.zeros_like(dd), qd)
    r = oracle.ffn_block("q4_0", tg.raw, tu.raw, wd0, gamma, 1e-5, x, d_model, ffn)
    assert np.array_equal(r["out"], x.astype(np.float64))
    td = synth.make_tensor("q4_0", d_model, ffn, rng)
    r = oracle.ffn_block("q4_0", tg.raw, tu.raw, td.raw, np.zeros(d_model, np.float32), 1e-5, x, d_model, ffn)
    assert np.array_equal(r["xn"], np.zeros_like(r["xn"]))
    assert np.array_equal(r["out"], x.astype(np.float64))
