"""GPU parity of the matrix-core path (every weight format, n_tok > 1) through the C ABI.

Bars (per element), with S = sum_j |w_ij x_tj| from the oracle:
  * y and the gate/up products: |y_gpu - y_ref| <= 8e-3 * S + 1e-7 (weights
    and x rounded to bf16, nearest even, fp32 accumulation);
  * inputs on which that rounding is exact (codes with power-of-two scales,
    small-integer x) and whose partial sums are exact in fp32: bit-identical
    to the oracle, under every tile shape -- this pins the column order the
    two operands share;
  * one-hot tokens: y[t][i] is the bf16 rounding (nearest even) of the
    oracle's weight w[i][c_t], bit for bit;
  * two runs bit-identical.
Shapes cover ragged rows (not a multiple of 16, 64 or 4), columns that leave a
partial 128-wide K step, token counts that leave a partial 16-token tile, and
every tile shape the library can launch.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu

# (rows, cols, n_tok)
SHAPES = [(1, 32, 2), (5, 96, 3), (150, 288, 17), (131, 576, 16), (64, 1536, 40), (97, 5120, 33),
          (300, 2048, 130), (40, 17408, 9)]
# (mtr, ntw, waves, run): every shape the override accepts (shapes the library
# does not build run as the nearest built one)
TILES = list(itertools.product((1, 2), (1, 2, 4, 8), (4, 8, 16), (1, 2, 4)))


def _pow2_q4_0(rows, cols, rng, lo=-4, hi=3):
    d = (2.0 ** rng.integers(lo, hi, (rows, cols // 32))).astype(np.float16)
    return synth.QTensor("w", "q4_0", rows, cols, synth.pack_q4_0(d, rng.integers(0, 16, (rows, cols))))


def _run(t, pk, x):
    return G.gemv_gpu(t, pk, x)


# Q4_K shapes: cols a multiple of 256 (ragged rows, partial K steps, partial token tiles)
SHAPES_K = [(1, 256, 2), (150, 768, 17), (64, 2048, 40), (97, 5632, 33), (300, 2048, 130), (40, 17408, 9)]


def _pow2_q4_k(rows, cols, rng):
    # d, dmin powers of two, sc a power of two, m = 0: every weight d*sc*q has
    # at most 4 significant bits (exact in bf16)
    nsb = cols // 256
    d = (2.0 ** rng.integers(-8, -5, (rows, nsb))).astype(np.float16)
    dmin = (2.0 ** rng.integers(-8, -5, (rows, nsb))).astype(np.float16)
    sc = (2 ** rng.integers(0, 6, (rows, nsb, 8))).astype(np.uint8)
    m = np.zeros((rows, nsb, 8), np.uint8)
    return synth.QTensor("w", "q4_k", rows, cols, synth.pack_q4_k(d, dmin, sc, m, rng.integers(0, 16, (rows, cols))))


@pytest.mark.parametrize("rows,cols,n_tok", SHAPES_K)
def test_prefill_q4_k_within_bound(rows, cols, n_tok):
    rng = np.random.default_rng(rows * 11 + cols + n_tok)
    t = synth.make_tensor("q4_k", rows, cols, rng)
    x = rng.standard_normal((n_tok, cols)).astype(np.float32)
    y = _run(t, G.upload(t), x)
    yr, S = oracle.gemv("q4_k", t.raw, x, rows, cols)
    G.check_bound(y, yr, S, rel=G.PF_REL, what=f"prefill q4_k {rows}x{cols} n_tok={n_tok}")


def test_prefill_q4_k_exact_inputs_bit_exact_every_tile():
    # weights exact in bf16 (see _pow2_q4_k: the minimum term is 0), small-integer
    # x: every partial sum is exact in fp32, under every tile shape
    rng = np.random.default_rng(1150)
    rows, cols, n_tok = 150, 1280, 37     # 40 sub-blocks: a partial K step for runs of 2 and 4
    t = _pow2_q4_k(rows, cols, rng)
    pk = G.upload(t)
    x = rng.integers(-3, 4, (n_tok, cols)).astype(np.float32)
    yr, _ = oracle.gemv("q4_k", t.raw, x, rows, cols)
    try:
        for tile in TILES:
            G.qg().set_prefill_override(*tile)
            y = _run(t, pk, x)
            assert np.array_equal(y.astype(np.float64), yr), f"q4_k tile (mtr, ntw, waves, run) = {tile}"
    finally:
        G.qg().set_prefill_override(0)


def test_prefill_q4_k_one_hot_tokens_give_bf16_weights():
    rng = np.random.default_rng(1350)
    rows, cols = 70, 2048
    t = synth.make_tensor("q4_k", rows, cols, rng)
    nb = cols // 32
    cs = np.array([32 * ((5 * k) % nb) + k for k in range(32)])
    x = np.zeros((32, cols), np.float32)
    x[np.arange(32), cs] = 1.0
    y = _run(t, G.upload(t), x)
    w32 = oracle.dequant("q4_k", t.raw, rows, cols)
    assert np.array_equal(y, G.bf16_rne(w32[:, cs]).T)


def test_prefill_q4_k_swiglu_ffn():
    # the TinyLlama-shaped Q4_K FFN at 24 tokens through swiglu_ffn, both
    # products on the matrix cores
    d_model, ffn = 2048, 5632
    rng = np.random.default_rng(1550)
    tens = [synth.make_tensor("q4_k", ffn, d_model, rng), synth.make_tensor("q4_k", ffn, d_model, rng),
            synth.make_tensor("q4_k", d_model, ffn, rng)]
    x = rng.standard_normal((24, d_model)).astype(np.float32)
    G.check_ffn("q4_k", tens, x, d_model, ffn, "ffn q4_k n_tok=24")


@pytest.mark.parametrize("rows,cols,n_tok", SHAPES)
def test_prefill_within_bound(rows, cols, n_tok):
    rng = np.random.default_rng(rows * 7 + cols + n_tok)
    t = synth.make_tensor("q4_0", rows, cols, rng)
    x = rng.standard_normal((n_tok, cols)).astype(np.float32)
    y = _run(t, G.upload(t), x)
    yr, S = oracle.gemv("q4_0", t.raw, x, rows, cols)
    G.check_bound(y, yr, S, rel=G.PF_REL, what=f"prefill {rows}x{cols} n_tok={n_tok}")


def test_prefill_integer_inputs_bit_exact_every_tile():
    # |(q-8) d x| <= 8 * 4 * 3 and every value a multiple of 2^-4: every
    # partial sum is exact in fp32, and bf16 holds every w and x exactly
    rng = np.random.default_rng(1100)
    rows, cols, n_tok = 150, 1056, 37     # 33 blocks: a partial K step
    t = _pow2_q4_0(rows, cols, rng)
    pk = G.upload(t)
    x = rng.integers(-3, 4, (n_tok, cols)).astype(np.float32)
    yr, _ = oracle.gemv("q4_0", t.raw, x, rows, cols)
    try:
        for tile in TILES:
            G.qg().set_prefill_override(*tile)
            y = _run(t, pk, x)
            assert np.array_equal(y.astype(np.float64), yr), f"tile (mtr, ntw, waves, run) = {tile}"
    finally:
        G.qg().set_prefill_override(0)


def test_prefill_gate_up_every_tile():
    # h = silu(Wg x) * (Wu x) with exact products: only the device's exp and
    # divide separate h from the oracle's
    rng = np.random.default_rng(1200)
    d_model, ffn, n_tok = 288, 200, 21
    tg, tu = _pow2_q4_0(ffn, d_model, rng, -6, -3), _pow2_q4_0(ffn, d_model, rng, -6, -3)
    pg, pu = G.upload(tg), G.upload(tu)
    x = rng.integers(-3, 4, (n_tok, d_model)).astype(np.float32)
    xd = G.torch.from_numpy(x).to(G.dev())
    r = {}
    r["g"], r["Sg"] = oracle.gemv("q4_0", tg.raw, x, ffn, d_model)
    r["u"], r["Su"] = oracle.gemv("q4_0", tu.raw, x, ffn, d_model)
    r["h"] = G.silu64(r["g"]) * r["u"]
    hb = G.h_bound(r, rel=0.0)
    try:
        for tile in TILES:
            G.qg().set_prefill_override(*tile)
            h = G.qg().swiglu_gate_up("q4_0", pg, pu, xd, d_model, ffn)
            G.torch.cuda.synchronize()
            h = h.cpu().numpy()
            assert np.all(np.abs(h - r["h"]) <= hb), f"tile (mtr, ntw, waves, run) = {tile}"
    finally:
        G.qg().set_prefill_override(0)


def test_prefill_one_hot_tokens_give_bf16_weights():
    # token t is one-hot at column 32*b_t + t: y[t][:] is column c_t of the
    # weights rounded to bf16; all 32 positions of a block are covered
    rng = np.random.default_rng(1300)
    rows, cols = 70, 2048
    t = synth.make_tensor("q4_0", rows, cols, rng)
    nb = cols // 32
    cs = np.array([32 * ((5 * k) % nb) + k for k in range(32)])
    x = np.zeros((32, cols), np.float32)
    x[np.arange(32), cs] = 1.0
    y = _run(t, G.upload(t), x)
    w32 = oracle.dequant("q4_0", t.raw, rows, cols).astype(np.float32)   # exact in fp32
    want = G.bf16_rne(w32[:, cs]).T
    assert np.array_equal(y, want)


def test_prefill_deterministic():
    rng = np.random.default_rng(1400)
    rows, cols, n_tok = 300, 5120, 64
    t = synth.make_tensor("q4_0", rows, cols, rng)
    pk = G.upload(t)
    x = rng.standard_normal((n_tok, cols)).astype(np.float32)
    assert np.array_equal(_run(t, pk, x), _run(t, pk, x))


def test_prefill_swiglu_ffn_batched():
    # SmolLM2-135M-shaped FFN block at 40 tokens, both products on the matrix cores
    d_model, ffn = 576, 1536
    rng = np.random.default_rng(1500)
    tens = [synth.make_tensor("q4_0", ffn, d_model, rng), synth.make_tensor("q4_0", ffn, d_model, rng),
            synth.make_tensor("q4_0", d_model, ffn, rng)]
    x = rng.standard_normal((40, d_model)).astype(np.float32)
    G.check_ffn("q4_0", tens, x, d_model, ffn, "ffn q4_0 n_tok=40")


def test_prefill_split_k_exact_and_deterministic():
    # K split over workgroups (partials in the scratch behind h, summed in
    # range order): with exact products, h is the same bit for bit for every
    # split, and each split's out stays within the bound and repeats exactly
    rng = np.random.default_rng(1600)
    d_model, ffn, n_tok = 1056, 800, 21     # 9 and 7 K steps: ragged ranges
    tg, tu = _pow2_q4_0(ffn, d_model, rng, -6, -3), _pow2_q4_0(ffn, d_model, rng, -6, -3)
    td = synth.make_tensor("q4_0", d_model, ffn, rng)
    pk = [G.upload(t) for t in (tg, tu, td)]
    x = rng.integers(-3, 4, (n_tok, d_model)).astype(np.float32)
    xd = G.torch.from_numpy(x).to(G.dev())
    r = {}
    r["g"], r["Sg"] = oracle.gemv("q4_0", tg.raw, x, ffn, d_model)
    r["u"], r["Su"] = oracle.gemv("q4_0", tu.raw, x, ffn, d_model)
    r["h"] = G.silu64(r["g"]) * r["u"]
    hb = G.h_bound(r, rel=0.0)
    po = (n_tok * ffn + 63) // 64 * 64
    scratch = G.torch.empty(po + 9 * 2 * n_tok * max(ffn, d_model), dtype=G.torch.float32, device=G.dev())
    h_ref = None
    try:
        for ks in (1, 2, 3, 4, 7, 9):
            G.qg().set_prefill_override(1, 2, 4, 1, ks)
            outs = []
            for _ in range(2):
                out, h = G.qg().swiglu_ffn("q4_0", pk[0], pk[1], pk[2], xd, d_model, ffn, h_scratch=scratch)
                G.torch.cuda.synchronize()
                outs.append(out.cpu().numpy())
                h = h.cpu().numpy()
            assert np.all(np.abs(h - r["h"]) <= hb), f"ksplit={ks}: h outside its bound"
            if h_ref is None:
                h_ref = h
            assert np.array_equal(h, h_ref), f"ksplit={ks}: h differs from the unsplit h"
            assert np.array_equal(outs[0], outs[1]), f"ksplit={ks}: not deterministic"
            yr, S = oracle.gemv("q4_0", td.raw, h, d_model, ffn)
            G.check_bound(outs[0], yr, S, rel=G.PF_REL, what=f"ksplit={ks} down")
    finally:
        G.qg().set_prefill_override(0)


def test_prefill_default_split_uses_scratch():
    # the built-in choice splits K for a narrow matrix at few tokens, and the
    # binding sizes the scratch for it
    ffn, d_model, n_tok = 17408, 512, 8
    elems = G.qg().swiglu_ffn_scratch_elems("q4_0", d_model, ffn, n_tok)
    assert elems > n_tok * ffn


def test_prefill_override_rejects_bad_shapes():
    for bad in ((3, 1, 4, 2, 0), (1, 3, 4, 2, 0), (1, 1, 2, 2, 0), (2, 16, 8, 2, 0), (1, 1, 4, 3, 0),
                (1, 1, 4, 8, 0), (1, 1, 4, 2, -1), (1, 1, 4, 2, 65)):
        assert G.qg().lib.qgemv_set_prefill_override(*bad) == -2, bad
    G.qg().set_prefill_override(0)



# Q6_K shapes: cols a multiple of 256 (ragged rows, partial K steps, partial token tiles)
SHAPES_6 = [(1, 256, 2), (150, 768, 17), (97, 5632, 33), (300, 2048, 130), (40, 5632, 9)]


def _pow2_q6_k(rows, cols, rng):
    # d and |sc| powers of two, codes 0..63: every weight d*sc*(q-32) has at
    # most 6 significant bits (exact in bf16); with x in -3..3 and at most
    # 1280 columns every partial sum stays below 2^14 in steps of 2^-8 (exact
    # in fp32)
    nsb = cols // 256
    d = (2.0 ** rng.integers(-8, -5, (rows, nsb))).astype(np.float16)
    sc = ((2 ** rng.integers(0, 4, (rows, nsb, 16))) * rng.choice([-1, 1], (rows, nsb, 16))).astype(np.int8)
    q = rng.integers(0, 64, (rows, cols))
    return synth.QTensor("w", "q6_k", rows, cols, synth.pack_q6_k(d, sc, q))


@pytest.mark.parametrize("rows,cols,n_tok", SHAPES_6)
def test_prefill_q6_k_within_bound(rows, cols, n_tok):
    rng = np.random.default_rng(rows * 13 + cols + n_tok)
    t = synth.make_tensor("q6_k", rows, cols, rng)
    x = rng.standard_normal((n_tok, cols)).astype(np.float32)
    y = _run(t, G.upload(t), x)
    yr, S = oracle.gemv("q6_k", t.raw, x, rows, cols)
    G.check_bound(y, yr, S, rel=G.PF_REL, what=f"prefill q6_k {rows}x{cols} n_tok={n_tok}")


def test_prefill_q6_k_exact_inputs_bit_exact_every_tile():
    rng = np.random.default_rng(1170)
    rows, cols, n_tok = 150, 1280, 37     # 40 blocks: a partial K step for runs of 2 and 4
    t = _pow2_q6_k(rows, cols, rng)
    pk = G.upload(t)
    x = rng.integers(-3, 4, (n_tok, cols)).astype(np.float32)
    yr, _ = oracle.gemv("q6_k", t.raw, x, rows, cols)
    try:
        for tile in TILES:
            G.qg().set_prefill_override(*tile)
            y = _run(t, pk, x)
            assert np.array_equal(y.astype(np.float64), yr), f"q6_k tile (mtr, ntw, waves, run) = {tile}"
    finally:
        G.qg().set_prefill_override(0)


def test_prefill_q6_k_one_hot_tokens_give_bf16_weights():
    # all 32 positions of a block (both halves, low and high nibbles, every
    # code word and high-bit shift)
    rng = np.random.default_rng(1370)
    rows, cols = 70, 2048
    t = synth.make_tensor("q6_k", rows, cols, rng)
    nb = cols // 32
    cs = np.array([32 * ((5 * k) % nb) + k for k in range(32)])
    x = np.zeros((32, cols), np.float32)
    x[np.arange(32), cs] = 1.0
    y = _run(t, G.upload(t), x)
    w32 = oracle.dequant("q6_k", t.raw, rows, cols).astype(np.float32)
    assert np.array_equal(y, G.bf16_rne(w32[:, cs]).T)


def test_prefill_q6_k_swiglu_ffn():
    # a Q6_K FFN at 24 tokens through swiglu_ffn, both products on the matrix cores
    d_model, ffn = 1024, 2816
    rng = np.random.default_rng(1570)
    tens = [synth.make_tensor("q6_k", ffn, d_model, rng), synth.make_tensor("q6_k", ffn, d_model, rng),
            synth.make_tensor("q6_k", d_model, ffn, rng)]
    x = rng.standard_normal((24, d_model)).astype(np.float32)
    G.check_ffn("q6_k", tens, x, d_model, ffn, "ffn q6_k n_tok=24")


# ---------------------------------------------------------------- 8-bit --
# Q8_0 and per-row INT8 on the matrix cores: the byte xor 0x80 read as a
# binary16 subnormal, then one fma, gives q*D exactly in fp32 (Q8_0: D = d;
# INT8: D = 1, the row scale multiplies the fp32 sums).
EIGHT = ("q8_0", "i8row")


def _pow2_8bit(fmt, rows, cols, rng):
    # every code -128..127 (the xor's edge included); Q8_0 d and INT8 row
    # scales powers of two: q*D has at most 8 significant bits (exact in bf16)
    q = rng.integers(-128, 128, (rows, cols)).astype(np.int8)
    if fmt == "q8_0":
        d = (2.0 ** rng.integers(-6, -2, (rows, cols // 32))).astype(np.float16)
        return synth.QTensor("w", "q8_0", rows, cols, synth.pack_q8_0(d, q))
    s = (2.0 ** rng.integers(-6, -2, rows)).astype(np.float32)
    return synth.QTensor("w", "i8row", rows, cols, q, row_scale=s)


@pytest.mark.parametrize("fmt", EIGHT)
@pytest.mark.parametrize("rows,cols,n_tok", SHAPES)
def test_prefill_8bit_within_bound(fmt, rows, cols, n_tok):
    rng = np.random.default_rng(rows * 7 + cols + n_tok + (5 if fmt == "i8row" else 0))
    t = synth.make_tensor(fmt, rows, cols, rng)
    x = rng.standard_normal((n_tok, cols)).astype(np.float32)
    y = _run(t, G.upload(t), x)
    yr, S = oracle.gemv(fmt, t.raw, x, rows, cols, row_scale=t.row_scale)
    G.check_bound(y, yr, S, rel=G.PF_REL, what=f"prefill {fmt} {rows}x{cols} n_tok={n_tok}")


@pytest.mark.parametrize("fmt", EIGHT)
def test_prefill_8bit_exact_inputs_bit_exact_every_tile(fmt):
    # |q*D*x| <= 128 * 2^-3 * 3 in steps of 2^-6: with 1312 columns every
    # partial sum is exact in fp32; 41 blocks leave a partial K step for
    # runs of 2 and 4
    rng = np.random.default_rng(1710 if fmt == "q8_0" else 1711)
    rows, cols, n_tok = 150, 1312, 37
    t = _pow2_8bit(fmt, rows, cols, rng)
    pk = G.upload(t)
    x = rng.integers(-3, 4, (n_tok, cols)).astype(np.float32)
    yr, _ = oracle.gemv(fmt, t.raw, x, rows, cols, row_scale=t.row_scale)
    try:
        for tile in TILES:
            G.qg().set_prefill_override(*tile)
            y = _run(t, pk, x)
            assert np.array_equal(y.astype(np.float64), yr), f"{fmt} tile (mtr, ntw, waves, run) = {tile}"
    finally:
        G.qg().set_prefill_override(0)


@pytest.mark.parametrize("fmt", EIGHT)
def test_prefill_8bit_one_hot_tokens(fmt):
    # all 32 positions of a block: Q8_0 gives the weight q*d rounded to bf16;
    # INT8 the fp32 weight q*s itself (the code is exact in bf16 and the
    # scale multiplies the fp32 sum)
    rng = np.random.default_rng(1720 if fmt == "q8_0" else 1721)
    rows, cols = 70, 2048
    t = synth.make_tensor(fmt, rows, cols, rng)
    nb = cols // 32
    cs = np.array([32 * ((5 * k) % nb) + k for k in range(32)])
    x = np.zeros((32, cols), np.float32)
    x[np.arange(32), cs] = 1.0
    y = _run(t, G.upload(t), x)
    w32 = oracle.dequant(fmt, t.raw, rows, cols, row_scale=t.row_scale).astype(np.float32)
    want = G.bf16_rne(w32[:, cs]).T if fmt == "q8_0" else w32[:, cs].T
    assert np.array_equal(y, want)


@pytest.mark.parametrize("fmt", EIGHT)
def test_prefill_8bit_swiglu_ffn(fmt):
    # a SmolLM2-135M-shaped FFN at 24 tokens through swiglu_ffn, both products
    # on the matrix cores
    d_model, ffn = 576, 1536
    rng = np.random.default_rng(1730 if fmt == "q8_0" else 1731)
    tens = [synth.make_tensor(fmt, ffn, d_model, rng), synth.make_tensor(fmt, ffn, d_model, rng),
            synth.make_tensor(fmt, d_model, ffn, rng)]
    x = rng.standard_normal((24, d_model)).astype(np.float32)
    G.check_ffn(fmt, tens, x, d_model, ffn, f"ffn {fmt} n_tok=24")


@pytest.mark.parametrize("fmt,n_tok", [("q4_0", 40), ("q4_0", 128), ("q6_k", 33), ("i8row", 64), ("q4_k", 32),
                                       ("q8_0", 35), ("q4_0", 8), ("q4_k", 13), ("i8row", 9)])
def test_swiglu_ffn_bf16_copies_bit_identical(fmt, n_tok):
    # from 8 tokens on with d_model * ffn >= 2^24, and the scratch
    # swiglu_ffn_scratch_elems asks for, both products read bf16 copies of x
    # and h made by a conversion launch; one float less of scratch keeps the
    # fp32 inputs. The copies round as the kernel does, so h and out are
    # bit-identical either way. (4096 x 4096: ragged token tiles, both copies)
    d_model, ffn = 4096, 4096
    rng = np.random.default_rng(1800 + n_tok)
    tens = [synth.make_tensor(fmt, ffn, d_model, rng), synth.make_tensor(fmt, ffn, d_model, rng),
            synth.make_tensor(fmt, d_model, ffn, rng)]
    pk = [G.upload(t) for t in tens]
    x = G.torch.from_numpy(rng.standard_normal((n_tok, d_model)).astype(np.float32)).to(G.dev())
    full = G.qg().swiglu_ffn_scratch_elems(fmt, d_model, ffn, n_tok)
    assert full > n_tok * ffn
    res = []
    for elems in (full, full - 1):
        sc = G.torch.full((elems,), float("nan"), device=G.dev())
        out, h = G.qg().swiglu_ffn(fmt, pk[0], pk[1], pk[2], x, d_model, ffn, h_scratch=sc)
        G.torch.cuda.synchronize()
        res.append((out.cpu().numpy(), h.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    # and the bf16-copy path (the default scratch) against the oracle (the
    # smaller batches: the oracle's time grows with the tokens)
    if n_tok <= 40:
        G.check_ffn(fmt, tens, x.cpu().numpy(), d_model, ffn, f"ffn {fmt} n_tok={n_tok} bf16 copies")


def test_swiglu_ffn_bf16_copies_graph_replays():
    # the matrix-core FFN with its bf16 copies, K split and conversion launch,
    # captured in a HIP graph and replayed three times with eager work and a
    # synchronization between the replays: every replay equals the eager call
    d_model, ffn, n_tok = 4096, 4096, 16
    rng = np.random.default_rng(1900)
    tens = [synth.make_tensor("q4_0", ffn, d_model, rng), synth.make_tensor("q4_0", ffn, d_model, rng),
            synth.make_tensor("q4_0", d_model, ffn, rng)]
    pk = [G.upload(t) for t in tens]
    torch = G.torch
    x = torch.from_numpy(rng.standard_normal((n_tok, d_model)).astype(np.float32)).to(G.dev())
    sc = torch.empty(G.qg().swiglu_ffn_scratch_elems("q4_0", d_model, ffn, n_tok), device=G.dev())
    out = torch.empty((n_tok, d_model), device=G.dev())
    G.qg().swiglu_ffn("q4_0", pk[0], pk[1], pk[2], x, d_model, ffn, out=out, h_scratch=sc)
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):   # the binding launches on torch's current stream: the capture stream
        G.qg().swiglu_ffn("q4_0", pk[0], pk[1], pk[2], x, d_model, ffn, out=out, h_scratch=sc)
    torch.cuda.synchronize()
    for k in range(3):
        out.fill_(float("nan"))
        sc.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {k}"
        G.qg().swiglu_ffn("q4_0", pk[0], pk[1], pk[2], x, d_model, ffn, out=torch.empty_like(out),
                          h_scratch=torch.empty_like(sc))   # eager work between the replays
        torch.cuda.synchronize()
