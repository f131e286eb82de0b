"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (per element):
  * dequantized weights: bit-identical to the oracle's fp32 values (+0 == -0);
  * y: |y_gpu - y_ref| <= 2e-5 * sum_j |w_ij x_j| + 1e-7 (fp32 accumulation);
  * special inputs whose exact result every summation order reaches (one-hot
    x, small-integer x with power-of-two scales): bit-identical;
  * determinism: two runs bit-identical.
Shapes span several workgroups, every lanes-per-row choice and ragged row
tails; the full-size workloads run in the launch configuration the bench uses.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu

FMTS = ["q4_0", "q8_0", "q4_k", "i8row", "q6_k"]
# (rows, cols): ragged rows, cols that pick 8/16/32/64 lanes per row
SHAPES = {
    "q4_0": [(1, 32), (7, 288), (131, 576), (200, 1536), (97, 5120), (33, 17408)],
    "q8_0": [(1, 32), (45, 576), (130, 2048), (67, 4096)],
    "q4_k": [(1, 256), (37, 2048), (129, 5632), (20, 4096)],
    "i8row": [(1, 32), (70, 2048), (131, 8192), (9, 96)],
    "q6_k": [(1, 256), (37, 2048), (129, 5632), (20, 4096), (33, 768)],
}


def _tensor(fmt, rows, cols, seed):
    return synth.make_tensor(fmt, rows, cols, np.random.default_rng(seed))


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_bit_exact(fmt):
    for k, (rows, cols) in enumerate(SHAPES[fmt]):
        t = _tensor(fmt, rows, cols, 100 + k)
        packed = G.upload(t)
        w = G.qg().qdequant(fmt, packed, rows, cols)
        G.torch.cuda.synchronize()
        ref = oracle.dequant(fmt, t.raw, rows, cols, row_scale=t.row_scale)
        got = w.cpu().numpy()
        assert np.array_equal(got, ref), (fmt, rows, cols)   # array_equal treats +0 == -0


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_within_bound(fmt):
    for k, (rows, cols) in enumerate(SHAPES[fmt]):
        t = _tensor(fmt, rows, cols, 200 + k)
        packed = G.upload(t)
        x = np.random.default_rng(300 + k).standard_normal(cols).astype(np.float32)
        y = G.gemv_gpu(t, packed, x)
        yr, S = oracle.gemv(fmt, t.raw, x, rows, cols, row_scale=t.row_scale)
        G.check_bound(y, yr, S, what=f"{fmt} {rows}x{cols}")


@pytest.mark.parametrize("fmt", FMTS)
def test_one_hot_x_gives_exact_column(fmt):
    rows, cols = {"q4_0": (77, 1536), "q8_0": (77, 576), "q4_k": (77, 2048), "i8row": (77, 2048),
                  "q6_k": (77, 2048)}[fmt]
    t = _tensor(fmt, rows, cols, 400)
    packed = G.upload(t)
    for k in (0, 1, 15, 16, 17, 31, 32, cols // 2 + 5, cols - 1):
        x = np.zeros(cols, np.float32)
        x[k] = 1.0
        y = G.gemv_gpu(t, packed, x)
        if fmt == "i8row":
            # y = s * q in one fp32 rounding
            want = (t.row_scale * t.raw[:, k].astype(np.float32)).astype(np.float32)
        else:
            want = oracle.dequant(fmt, t.raw, rows, cols)[:, k]
        assert np.array_equal(y, want), (fmt, k)


def _pow2_tensor(fmt, rows, cols, rng):
    """Codes from the generator's distributions, scales powers of two."""
    if fmt == "q4_0":
        d = (2.0 ** rng.integers(-6, -2, (rows, cols // 32))).astype(np.float16)
        return synth.pack_q4_0(d, rng.integers(0, 16, (rows, cols)))
    if fmt == "q8_0":
        d = (2.0 ** rng.integers(-8, -4, (rows, cols // 32))).astype(np.float16)
        return synth.pack_q8_0(d, rng.integers(-127, 128, (rows, cols)).astype(np.int8))
    if fmt == "q4_k":
        nsb = cols // 256
        d = (2.0 ** rng.integers(-10, -8, (rows, nsb))).astype(np.float16)
        dmin = (2.0 ** rng.integers(-10, -8, (rows, nsb))).astype(np.float16)
        return synth.pack_q4_k(d, dmin, rng.integers(0, 64, (rows, nsb, 8)), rng.integers(0, 64, (rows, nsb, 8)),
                               rng.integers(0, 16, (rows, cols)))
    if fmt == "q6_k":
        # |d * sc * (q - 32)| <= 2^-9 * 8 * 32: partial sums stay multiples of
        # 2^-10 far below 2^14
        nsb = cols // 256
        d = (2.0 ** rng.integers(-10, -8, (rows, nsb))).astype(np.float16)
        return synth.pack_q6_k(d, rng.integers(-8, 9, (rows, nsb, 16)).astype(np.int8),
                               rng.integers(0, 64, (rows, cols)))
    raise ValueError(fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_integer_inputs_bit_exact(fmt):
    # x in {-2..2} and power-of-two scales: every partial sum is exactly
    # representable, so any summation order gives the oracle's value exactly
    rng = np.random.default_rng(500)
    rows, cols = 150, 1024
    if fmt == "i8row":
        q = rng.integers(-127, 128, (rows, cols)).astype(np.int8)
        s = (2.0 ** rng.integers(-12, -8, rows)).astype(np.float32)
        t = synth.QTensor("w", fmt, rows, cols, q, row_scale=s)
    else:
        t = synth.QTensor("w", fmt, rows, cols, _pow2_tensor(fmt, rows, cols, rng))
    packed = G.upload(t)
    x = rng.integers(-2, 3, cols).astype(np.float32)
    y = G.gemv_gpu(t, packed, x)
    yr, _ = oracle.gemv(fmt, t.raw, x, rows, cols, row_scale=t.row_scale)
    assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("fmt", FMTS)
def test_determinism_and_power_of_two_linearity(fmt):
    rows, cols = {"q4_0": (300, 5120), "q8_0": (300, 576), "q4_k": (300, 2048), "i8row": (300, 2048),
                  "q6_k": (300, 5632)}[fmt]
    t = _tensor(fmt, rows, cols, 600)
    packed = G.upload(t)
    x = np.random.default_rng(601).standard_normal(cols).astype(np.float32)
    y1 = G.gemv_gpu(t, packed, x)
    y2 = G.gemv_gpu(t, packed, x)
    y8 = G.gemv_gpu(t, packed, x * np.float32(8.0))
    assert np.array_equal(y1, y2)
    assert np.array_equal(y8, np.float32(8.0) * y1)


@pytest.mark.parametrize("fmt", FMTS)
def test_batched_tokens_match_single(fmt):
    rows, cols = {"q4_0": (96, 576), "q8_0": (96, 576), "q4_k": (96, 2048), "i8row": (96, 2048),
                  "q6_k": (96, 2048)}[fmt]
    t = _tensor(fmt, rows, cols, 700)
    packed = G.upload(t)
    x = np.random.default_rng(701).standard_normal((5, cols)).astype(np.float32)
    yb = G.gemv_gpu(t, packed, x)
    yr, S = oracle.gemv(fmt, t.raw, x, rows, cols, row_scale=t.row_scale)
    G.check_bound(yb, yr, S, rel=G.rel_for(fmt, 5), what=f"{fmt} n_tok=5")
    if fmt == "q4_0":
        # the matrix-core path switched off: the GEMV loop, fp32 bound
        try:
            G.qg().set_prefill_override(-1)
            G.check_bound(G.gemv_gpu(t, packed, x), yr, S, what=f"{fmt} n_tok=5 GEMV loop")
        finally:
            G.qg().set_prefill_override(0)
    for k in range(5):
        G.check_bound(G.gemv_gpu(t, packed, x[k]), yr[k], S[k], what=f"{fmt} token {k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_every_launch_shape(fmt):
    # every lanes-per-row / rows-per-group / waves / prefetch-depth choice the
    # tuning hook allows, with and without a grid-stride workgroup cap
    rows, cols = 203, {"q4_0": 1536, "q8_0": 1536, "q4_k": 2048, "i8row": 1536, "q6_k": 2048}[fmt]
    t = _tensor(fmt, rows, cols, 800)
    packed = G.upload(t)
    x = np.random.default_rng(801).standard_normal(cols).astype(np.float32)
    yr, S = oracle.gemv(fmt, t.raw, x, rows, cols, row_scale=t.row_scale)
    try:
        for lpr in (8, 16, 32, 64):
            for r in (1, 2):
                for waves in (1, 3, 4, 5, 8):
                    for depth in (2, 4):
                        for max_wg in (0, 3):
                            for cpl in (1, 2, 4):
                                G.qg().set_launch_override(lpr, r, waves, depth, max_wg, cpl)
                                y = G.gemv_gpu(t, packed, x)
                                G.check_bound(y, yr, S, what=f"{fmt} lpr={lpr} r={r} waves={waves} "
                                                             f"depth={depth} max_wg={max_wg} cpl={cpl}")
    finally:
        G.qg().set_launch_override(0)


@pytest.mark.parametrize("fmt", FMTS)
def test_gate_up_every_launch_shape(fmt):
    d_model, ffn = (2048, 203) if fmt in ("q4_k", "q6_k") else (1536, 203)   # ragged ffn rows
    rng = np.random.default_rng(850)
    g = synth.make_tensor(fmt, ffn, d_model, rng)
    u = synth.make_tensor(fmt, ffn, d_model, rng)
    pg, pu = G.upload(g), G.upload(u)
    x = np.random.default_rng(851).standard_normal((1, d_model)).astype(np.float32)
    r = {}
    r["g"], r["Sg"] = oracle.gemv(fmt, g.raw, x, ffn, d_model, row_scale=g.row_scale)
    r["u"], r["Su"] = oracle.gemv(fmt, u.raw, x, ffn, d_model, row_scale=u.row_scale)
    r["h"] = np.array([[oracle.silu(v) for v in r["g"][0]]]) * r["u"]
    hb = G.h_bound(r)
    xd = G.torch.from_numpy(x).to(G.dev())
    try:
        for lpr in (8, 16, 32, 64):
            for rr in (1, 2):
                for waves in (1, 3, 4, 5, 8):
                    for depth in (2, 4):
                        for max_wg in (0, 3):
                            for cpl in (1, 2, 4):
                                G.qg().set_launch_override(lpr, rr, waves, depth, max_wg, cpl)
                                h = G.qg().swiglu_gate_up(fmt, pg, pu, xd, d_model, ffn)
                                G.torch.cuda.synchronize()
                                err = np.abs(h.cpu().numpy() - r["h"])
                                assert np.all(err <= hb), (fmt, lpr, rr, waves, depth, max_wg, cpl)
    finally:
        G.qg().set_launch_override(0)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_grouped_scales_with_odd_chunk_rows(fmt):
    # 288 columns = 9 chunks per row: grouped scale loads must not be used
    rows, cols = 77, 288
    t = _tensor(fmt, rows, cols, 870)
    packed = G.upload(t)
    x = np.random.default_rng(871).standard_normal(cols).astype(np.float32)
    yr, S = oracle.gemv(fmt, t.raw, x, rows, cols, row_scale=t.row_scale)
    try:
        for cpl in (2, 4):
            G.qg().set_launch_override(8, 1, 4, 2, 0, cpl)
            G.check_bound(G.gemv_gpu(t, packed, x), yr, S, what=f"{fmt} cpl={cpl} 9 chunks")
    finally:
        G.qg().set_launch_override(0)


def test_q6_k_neutral_codes_give_exact_zero():
    # every code 32: w = 0 whatever d and the scales; the offset is folded in
    # through the staged half-chunk sums, summed in the codes' own order, so
    # the products cancel exactly for any x (under every launch shape)
    rows, cols = 75, 2048
    rng = np.random.default_rng(880)
    d, sc, _ = synth.draw_q6_k(rng, rows, cols)
    t = synth.QTensor("w", "q6_k", rows, cols, synth.pack_q6_k(d, sc, np.full((rows, cols), 32)))
    packed = G.upload(t)
    x = (100.0 * rng.standard_normal(cols)).astype(np.float32)
    assert np.all(G.gemv_gpu(t, packed, x) == 0)
    try:
        for lpr, cpl in ((8, 1), (16, 2), (32, 2), (64, 1)):
            G.qg().set_launch_override(lpr, 2, 4, 2, 0, cpl)
            assert np.all(G.gemv_gpu(t, packed, x) == 0), (lpr, cpl)
    finally:
        G.qg().set_launch_override(0)


# ----------------------------------------------------------------- SwiGLU --
def _ffn_tensors(fmt, d_model, ffn, seed):
    rng = np.random.default_rng(seed)
    return [synth.make_tensor(fmt, ffn, d_model, rng), synth.make_tensor(fmt, ffn, d_model, rng),
            synth.make_tensor(fmt, d_model, ffn, rng)]


@pytest.mark.parametrize("fmt", FMTS)
def test_swiglu_small(fmt):
    d_model, ffn = (256, 768) if fmt in ("q4_k", "q6_k") else (288, 768)
    tens = _ffn_tensors(fmt, d_model, ffn, 900)
    x = np.random.default_rng(901).standard_normal((1, d_model)).astype(np.float32)
    out, h, r, hb = G.check_ffn(fmt, tens, x, d_model, ffn, f"ffn {fmt}")
    # end to end: the h error propagated through |Wd|
    wd = np.abs(oracle.dequant(fmt, tens[2].raw, d_model, ffn, row_scale=tens[2].row_scale).astype(np.float64))
    bound = G.REL * r["Sd"] + wd @ hb[0] + G.ABS
    assert np.all(np.abs(out - r["out"]) <= bound)


def test_swiglu_batched_tokens():
    d_model, ffn = 288, 768
    tens = _ffn_tensors("q4_0", d_model, ffn, 950)
    x = np.random.default_rng(951).standard_normal((3, d_model)).astype(np.float32)
    G.check_ffn("q4_0", tens, x, d_model, ffn, "ffn q4_0 n_tok=3")


def test_swiglu_zero_gate_gives_zero():
    d_model, ffn = 288, 768
    rng = np.random.default_rng(960)
    dg, qg_ = synth.draw_q4_0(rng, ffn, d_model)
    tg = synth.QTensor("g", "q4_0", ffn, d_model, synth.pack_q4_0(np.zeros_like(dg), qg_))
    tu = synth.make_tensor("q4_0", ffn, d_model, rng)
    td = synth.make_tensor("q4_0", d_model, ffn, rng)
    pk = [G.upload(t) for t in (tg, tu, td)]
    xd = G.torch.from_numpy(rng.standard_normal((1, d_model)).astype(np.float32)).to(G.dev())
    out, h = G.qg().swiglu_ffn("q4_0", pk[0], pk[1], pk[2], xd, d_model, ffn)
    G.torch.cuda.synchronize()
    assert G.torch.all(h == 0) and G.torch.all(out == 0)
