"""GPU parity at the edges of the scale encodings, and the bf16 rounding of x.

Scales: the binary16 d (and Q4_K's dmin) of every format drawn over every
binade -- negative values, subnormals (0x0001 and 0x03ff among them), +0 and
-0, values next to 65504 -- and per-row INT8 fp32 scales over the whole
exponent range (subnormals, zeros, both signs).  The oracle decodes binary16
by its definition (sign, 5-bit exponent, 10-bit fraction, subnormals m*2^-24)
and forms each weight exactly (the block definitions in the llmoxide blog,
section 10, and the llamini.cpp post, "What I reimplemented"); nothing is
flushed to zero on either side.  Checked:
  * qdequant bit-identical to the oracle (+0 == -0);
  * one-hot x on the GEMV path: y is the weight column itself, bit for bit;
    one-hot tokens on the matrix cores: y is its bf16 rounding (INT8: the
    fp32 weight, whose row scale multiplies the fp32 sum);
  * random x: both paths within their bounds (2e-5 and 8e-3 of sum |w x|).
Q8_0 codes span -128..127 (one row all -128).

bf16 rounding of x on the matrix cores: one-hot tokens whose value sits
between two bf16 neighbours -- exact ties with an even and an odd lower
neighbour, one unit either side of a tie, the top of an interval -- give
y = bf16(w) * bf16(v) exactly (two 8-bit significands: an exact fp32
product), so a truncating or ties-away conversion fails.  The same values
through swiglu_ffn with its bf16 copy of x (the conversion launch) give
h = silu(g) u with g and u exact single products.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu

FMTS = ["q4_0", "q8_0", "q4_k", "i8row", "q6_k"]
F16_SPECIAL = [0x0001, 0x03FF, 0x0400, 0x8001, 0x83FF, 0x0000, 0x8000, 0x7BFF, 0xFBFF, 0x7BFE, 0x3C00, 0xBC00,
               0x0200, 0x8200]


def edge_f16(rng, shape):
    """binary16 values over every binade (exponent field 0..30, any fraction,
    either sign), with the special values above at random places."""
    bits = (rng.integers(0, 2, shape) << 15) | (rng.integers(0, 31, shape) << 10) | rng.integers(0, 1024, shape)
    flat = bits.reshape(-1)
    pos = rng.choice(flat.size, size=min(flat.size, 4 * len(F16_SPECIAL)), replace=False)
    flat[pos] = np.resize(F16_SPECIAL, pos.size)
    return flat.reshape(shape).astype(np.uint16).view(np.float16)


def row_binade_f16(rng, shape):
    """binary16 scales whose rows each keep to one binade (random sign, some
    +-0), the binades running from subnormal to the top: per-row sums of
    |w x| are then not dominated by one block, so the bound tests see every
    row's magnitude."""
    rows = shape[0]
    e = np.resize(np.arange(31), rows)[:, None]
    bits = (rng.integers(0, 2, shape) << 15) | (e << 10) | rng.integers(0, 1024, shape)
    z = rng.random(shape) < 0.05
    bits[z] = rng.choice([0x0000, 0x8000], size=int(z.sum()))
    return bits.astype(np.uint16).view(np.float16)


def edge_f32_scales(rng, n, per_row_binades=False):
    """fp32 row scales: subnormals, +-0, both signs, exponents up to 2^99."""
    e = np.resize(np.arange(0, 227), n) if per_row_binades else rng.integers(0, 227, n)
    bits = (rng.integers(0, 2, n) << 31) | (e << 23) | rng.integers(0, 1 << 23, n)
    bits[: min(n, 4)] = [0x00000001, 0x007FFFFF, 0x00000000, 0x80000000][: min(n, 4)]
    return bits.astype(np.uint32).view(np.float32)


def make(fmt, rows, cols, rng, scales):
    """A tensor of format fmt whose scales come from `scales(rng, shape)`
    (binary16) or, for INT8 rows, from edge_f32_scales."""
    if fmt == "q4_0":
        return synth.QTensor("w", fmt, rows, cols, synth.pack_q4_0(scales(rng, (rows, cols // 32)),
                                                                   rng.integers(0, 16, (rows, cols))))
    if fmt == "q8_0":
        q = rng.integers(-128, 128, (rows, cols)).astype(np.int8)
        q[rows // 2] = -128
        return synth.QTensor("w", fmt, rows, cols, synth.pack_q8_0(scales(rng, (rows, cols // 32)), q))
    if fmt == "q4_k":
        nsb = cols // 256
        return synth.QTensor("w", fmt, rows, cols, synth.pack_q4_k(
            scales(rng, (rows, nsb)), scales(rng, (rows, nsb)), rng.integers(0, 64, (rows, nsb, 8)),
            rng.integers(0, 64, (rows, nsb, 8)), rng.integers(0, 16, (rows, cols))))
    if fmt == "q6_k":
        nsb = cols // 256
        return synth.QTensor("w", fmt, rows, cols, synth.pack_q6_k(
            scales(rng, (rows, nsb)), rng.integers(-128, 128, (rows, nsb, 16)).astype(np.int8),
            rng.integers(0, 64, (rows, cols))))
    q = rng.integers(-128, 128, (rows, cols)).astype(np.int8)
    return synth.QTensor("w", fmt, rows, cols, q,
                         row_scale=edge_f32_scales(rng, rows, per_row_binades=scales is row_binade_f16))


SHAPE = {"q4_0": (131, 2048), "q8_0": (131, 2048), "q4_k": (131, 2048), "i8row": (131, 2048), "q6_k": (131, 2048)}


@pytest.mark.parametrize("fmt", FMTS)
def test_edge_scales_dequant_bit_exact(fmt):
    rows, cols = SHAPE[fmt]
    t = make(fmt, rows, cols, np.random.default_rng(3100 + FMTS.index(fmt)), edge_f16)
    w = G.qg().qdequant(fmt, G.upload(t), rows, cols)
    G.torch.cuda.synchronize()
    ref = oracle.dequant(fmt, t.raw, rows, cols, row_scale=t.row_scale)
    assert np.array_equal(w.cpu().numpy(), ref)


def _weights32(t):
    return oracle.dequant(t.fmt, t.raw, t.rows, t.cols, row_scale=t.row_scale).astype(np.float32)


@pytest.mark.parametrize("fmt", FMTS)
def test_edge_scales_gemv_one_hot_every_block(fmt):
    # one-hot x at one column of every block (a different position in each),
    # one GEMV launch per token: y is that weight column, bit for bit
    rows, cols = SHAPE[fmt]
    t = make(fmt, rows, cols, np.random.default_rng(3200 + FMTS.index(fmt)), edge_f16)
    pk = G.upload(t)
    w32 = _weights32(t)
    nb = cols // 32
    cs = np.array([32 * b + (7 * b) % 32 for b in range(nb)])
    x = np.zeros((nb, cols), np.float32)
    x[np.arange(nb), cs] = 1.0
    try:
        G.qg().set_prefill_override(-1)   # the per-token GEMV for every token
        y = G.gemv_gpu(t, pk, x)
    finally:
        G.qg().set_prefill_override(0)
    assert np.array_equal(y, w32[:, cs].T)


@pytest.mark.parametrize("fmt", FMTS)
def test_edge_scales_matrix_cores_one_hot_every_block(fmt):
    # the same columns as tokens of one matrix-core product: y is the bf16
    # rounding of each weight (INT8: the fp32 weight q*s)
    rows, cols = SHAPE[fmt]
    t = make(fmt, rows, cols, np.random.default_rng(3300 + FMTS.index(fmt)), edge_f16)
    w32 = _weights32(t)
    nb = cols // 32
    cs = np.array([32 * b + (11 * b) % 32 for b in range(nb)])
    x = np.zeros((nb, cols), np.float32)
    x[np.arange(nb), cs] = 1.0
    y = G.gemv_gpu(t, G.upload(t), x)
    want = w32[:, cs].T if fmt == "i8row" else G.bf16_rne(w32[:, cs]).T
    assert np.array_equal(y, want)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n_tok", [1, 5])
def test_edge_scales_within_bound(fmt, n_tok):
    # random x, every row's scales in one binade (subnormal to 2^15, either
    # sign, some zeros): the GEMV (1 token) and the matrix cores (5 tokens)
    rows, cols = SHAPE[fmt]
    rng = np.random.default_rng(3400 + 10 * FMTS.index(fmt) + n_tok)
    t = make(fmt, rows, cols, rng, row_binade_f16)
    x = rng.standard_normal((n_tok, cols)).astype(np.float32)
    y = G.gemv_gpu(t, G.upload(t), x)
    yr, S = oracle.gemv(fmt, t.raw, x, rows, cols, row_scale=t.row_scale)
    G.check_bound(y, yr, S, rel=G.rel_for(fmt, n_tok), what=f"{fmt} edge scales n_tok={n_tok}")


# fp32 values between bf16 neighbours: upper 16 bits (the bf16 below) and lower 16 bits
_HI = [0x3F80, 0x3F81, 0xBF80, 0xBF81, 0x4049, 0x404A, 0x3E00, 0xC2FF]
_LO = [0x8000, 0x7FFF, 0x8001, 0xFFFF, 0x0001, 0xC000]


def rne_probe_values():
    v = np.array([(h << 16) | l for h in _HI for l in _LO], dtype=np.uint32).view(np.float32)
    # the probe's worth: truncation and ties-away each disagree with nearest even on some of these
    r = G.bf16_rne(v)
    trunc = (v.view(np.uint32) & 0xFFFF0000).view(np.float32)
    away = ((v.view(np.uint32) + 0x8000) & 0xFFFF0000).view(np.float32)
    assert (r != trunc).any() and (r != away).any()
    return v


@pytest.mark.parametrize("fmt", FMTS)
def test_matrix_cores_round_x_to_bf16_nearest_even(fmt):
    rows, cols = 70, 2048
    rng = np.random.default_rng(3500 + FMTS.index(fmt))
    t = synth.make_tensor(fmt, rows, cols, rng)
    v = rne_probe_values()
    n = v.size
    cs = rng.choice(cols, size=n, replace=False)
    x = np.zeros((n, cols), np.float32)
    x[np.arange(n), cs] = v
    y = G.gemv_gpu(t, G.upload(t), x)
    w32 = _weights32(t)[:, cs].T                     # [n][rows]
    vb = G.bf16_rne(v)[:, None]
    if fmt == "i8row":
        q = t.raw[:, cs].T.astype(np.float32)        # the codes are exact in bf16
        want = (t.row_scale[None, :] * (q * vb)).astype(np.float32)
    else:
        want = (G.bf16_rne(w32) * vb).astype(np.float32)   # 8-bit by 8-bit significands: exact
    assert np.array_equal(y, want)


def test_ffn_bf16_copy_of_x_rounds_nearest_even():
    # 2048 x 8192 at 8 tokens: swiglu_ffn converts x to bf16 in its scratch
    # (one launch) and both gate and up read that copy; one-hot tokens make g
    # and u single exact products of bf16 values, so h = silu(g) u to the
    # device silu's budget
    d_model, ffn, n_tok = 2048, 8192, 8
    assert G.qg().swiglu_ffn_scratch_elems("q4_0", d_model, ffn, n_tok) > n_tok * ffn   # the copies are made
    rng = np.random.default_rng(3600)
    tens = [synth.make_tensor("q4_0", ffn, d_model, rng), synth.make_tensor("q4_0", ffn, d_model, rng),
            synth.make_tensor("q4_0", d_model, ffn, rng)]
    pk = [G.upload(t) for t in tens]
    v = rne_probe_values()
    sel = [k for k in range(v.size) if G.bf16_rne(v[k:k + 1])[0] != (v[k:k + 1].view(np.uint32) & 0xFFFF0000)
           .view(np.float32)[0]][:n_tok]                 # values truncation would get wrong
    v = v[sel]
    cs = rng.choice(d_model, size=n_tok, replace=False)
    x = np.zeros((n_tok, d_model), np.float32)
    x[np.arange(n_tok), cs] = v
    out, h = G.qg().swiglu_ffn("q4_0", pk[0], pk[1], pk[2], G.torch.from_numpy(x).to(G.dev()), d_model, ffn)
    G.torch.cuda.synchronize()
    h = h.cpu().numpy().astype(np.float64)
    vb = G.bf16_rne(v)[:, None].astype(np.float64)
    g = G.bf16_rne(_weights32(tens[0])[:, cs].T).astype(np.float64) * vb
    u = G.bf16_rne(_weights32(tens[1])[:, cs].T).astype(np.float64) * vb
    want = G.silu64(g) * u
    assert np.all(np.abs(h - want) <= G.SILU_REL * np.abs(want) + 1e-30)
