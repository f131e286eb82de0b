"""Pins for the oracle's SwiGLU FFN (g = Wg x, u = Wu x, h = silu(g) u, out = Wd h).

* SiLU at hand-worked points and the identity silu(g) - silu(-g) = g;
  comparison with scipy's logistic function (x * expit(x), the product form);
* zero gate scales or zero up scales give h = 0 and out = 0 exactly;
* identity-pattern Q8_0 matrices turn the FFN into the closed form
  out = silu(x) * x, elementwise.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth
from tests import _golden as G


def test_silu_golden_and_identities():
    for x, want, _ in G.load("silu_values.json")["cases"]:
        assert abs(oracle.silu(x) - want) <= 2e-16 * max(1.0, abs(want))
    for g in np.linspace(-30, 30, 241):
        assert abs((oracle.silu(g) - oracle.silu(-g)) - g) <= 1e-14 * max(1.0, abs(g))
        assert abs(oracle.silu(g) - g * expit(g)) <= 1e-15 * max(1.0, abs(g))
    assert oracle.silu(60.0) == 60.0
    assert abs(oracle.silu(-60.0)) < 1e-24


def _identity_q8(n, cols, d_bits=0x3C00):
    """[n][cols] Q8_0 with code 1 on the diagonal, scale 1."""
    q = np.zeros((n, cols), np.int8)
    for i in range(min(n, cols)):
        q[i, i] = 1
    d = np.full((n, cols // 32), np.uint16(d_bits)).view(np.float16)
    return synth.pack_q8_0(d, q)


def test_identity_ffn_closed_form():
    n = 64
    eye = _identity_q8(n, n)
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, n)).astype(np.float32)
    r = oracle.swiglu("q8_0", eye, eye, eye, x, n, n)
    x64 = x.astype(np.float64)
    assert np.array_equal(r["g"], x64) and np.array_equal(r["u"], x64)
    want = x64 * x64 * expit(x64)
    assert np.all(np.abs(r["out"] - want) <= 1e-15 * np.maximum(1, np.abs(want)))
    assert np.array_equal(r["h"], r["out"])


def test_gate_and_up_roles_are_distinct():
    # gate = x, up = 2x (scale 2): h = silu(x) * 2x, not silu(2x) * x
    n = 32
    rng = np.random.default_rng(24)
    x = rng.standard_normal((2, n)).astype(np.float32)
    r = oracle.swiglu("q8_0", _identity_q8(n, n), _identity_q8(n, n, 0x4000), _identity_q8(n, n), x, n, n)
    x64 = x.astype(np.float64)
    want = x64 * expit(x64) * 2 * x64
    assert np.all(np.abs(r["h"] - want) <= 1e-15 * np.maximum(1, np.abs(want)))


@pytest.mark.parametrize("which", ["gate", "up"])
def test_zero_scale_branch_kills_output(which):
    rng = np.random.default_rng(22)
    d_model, ffn = 64, 96
    dg, qg = synth.draw_q4_0(rng, ffn, d_model)
    du, qu = synth.draw_q4_0(rng, ffn, d_model)
    dd, qd = synth.draw_q4_0(rng, d_model, ffn)
    if which == "gate":
        dg = np.zeros_like(dg)
    else:
        du = np.zeros_like(du)
    x = rng.standard_normal((2, d_model)).astype(np.float32)
    r = oracle.swiglu("q4_0", synth.pack_q4_0(dg, qg), synth.pack_q4_0(du, qu),
                      synth.pack_q4_0(dd, qd), x, d_model, ffn)
    assert np.all(r["h"] == 0) and np.all(r["out"] == 0)


def test_i8row_swiglu_runs_with_row_scales():
    rng = np.random.default_rng(23)
    d_model, ffn = 32, 48
    g = synth.make_tensor("i8row", ffn, d_model, rng)
    u = synth.make_tensor("i8row", ffn, d_model, rng)
    d = synth.make_tensor("i8row", d_model, ffn, rng)
    x = rng.standard_normal((1, d_model)).astype(np.float32)
    r = oracle.swiglu("i8row", g.raw, u.raw, d.raw, x, d_model, ffn, g.row_scale, u.row_scale, d.row_scale)
    yg, _ = oracle.gemv("i8row", g.raw, x, ffn, d_model, row_scale=g.row_scale)
    assert np.array_equal(r["g"], yg)
    assert np.all(np.isfinite(r["out"]))
