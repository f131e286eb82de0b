"""GPU parity of the FFN block of the residual stream through the C ABI:
out = x + Wd (silu(Wg xn) * (Wu xn)), xn = rmsnorm(x) * gamma (llmoxide blog,
sections 4 and 7), against oracle.ffn_block.

Stage-wise bars, S from the oracle:
  * h against silu(g) u of the oracle's normalized input, within the
    first-order propagation of the product bounds of g and u; each of those
    bounds gets a relative 4e-6 for the fp32 RMSNorm scale (a sum of squares
    over at most ~100 sequential roundings, a square root and a division);
  * out against x + (the oracle's down product of the device's own h), within
    the product bound plus the final add's rounding (2^-24 |out|);
  * out == x exactly when the down scales are 0; in place (out is x) equals
    out of place bit for bit where both run the same form (out of place,
    Q4_0 rows of 256 blocks and more run the down product in K halves, whose
    summation order differs: test_gpu_khalf covers that form).
Formats: all four on the GEMV path (norm fused into the gate/up staging,
residual into the down epilogue); Q4_0 with several tokens on the matrix cores.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu

NORM_REL = 4e-6
EPS = 1e-5


def _tensors(fmt, d_model, ffn, seed):
    rng = np.random.default_rng(seed)
    return [synth.make_tensor(fmt, ffn, d_model, rng), synth.make_tensor(fmt, ffn, d_model, rng),
            synth.make_tensor(fmt, d_model, ffn, rng)]


def _run(fmt, tens, pk, gamma, x, d_model, ffn, out=None, in_place=False):
    xd = G.torch.from_numpy(np.ascontiguousarray(x)).to(G.dev())
    gd = G.torch.from_numpy(gamma).to(G.dev())
    o = xd if in_place else out
    o, h = G.qg().swiglu_ffn_block(fmt, pk[0], pk[1], pk[2], gd, EPS, xd, d_model, ffn, out=o)
    G.torch.cuda.synchronize()
    return o.cpu().numpy(), h.cpu().numpy()


def check_block(fmt, tens, x, gamma, d_model, ffn, what):
    g, u, d = tens
    pk = [G.upload(t) for t in tens]
    out, h = _run(fmt, tens, pk, gamma, x, d_model, ffn)
    r = oracle.ffn_block(fmt, g.raw, u.raw, d.raw, gamma, EPS, x, d_model, ffn, g.row_scale, u.row_scale,
                         d.row_scale)
    rel = G.rel_for(fmt, x.shape[0])
    hb = G.h_bound(r, rel + NORM_REL)
    assert np.all(np.abs(h - r["h"]) <= hb), f"{what}: h outside its bound"
    yr, S = oracle.gemv(fmt, d.raw, h, d_model, ffn, row_scale=d.row_scale)
    want = x.astype(np.float64) + yr
    bound = rel * S + G.ABS + np.abs(want) * 2.0 ** -24
    assert np.all(np.abs(out - want) <= bound), f"{what}: out outside its bound"
    return pk, out


@pytest.mark.parametrize("fmt,n_tok", [("q4_0", 1), ("q8_0", 1), ("q4_k", 1), ("i8row", 1), ("q6_k", 1), ("q8_0", 3),
                                       ("q4_0", 3), ("q4_0", 40), ("q6_k", 2), ("q4_k", 3), ("q4_k", 20),
                                       ("q8_0", 20), ("i8row", 3), ("i8row", 20), ("q6_k", 20)])
def test_block_matches_oracle(fmt, n_tok):
    d_model, ffn = (256, 768) if fmt in ("q4_k", "q6_k") else (288, 768)
    tens = _tensors(fmt, d_model, ffn, 2000 + n_tok)
    rng = np.random.default_rng(2100 + n_tok)
    x = (3.0 * rng.standard_normal((n_tok, d_model))).astype(np.float32)
    gamma = rng.uniform(0.2, 2.0, d_model).astype(np.float32)
    check_block(fmt, tens, x, gamma, d_model, ffn, f"block {fmt} n_tok={n_tok}")


@pytest.mark.parametrize("fmt,n_tok", [("q4_0", 1), ("i8row", 1), ("q4_0", 24)])
def test_block_in_place_equals_out_of_place(fmt, n_tok):
    d_model, ffn = 576, 1536
    tens = _tensors(fmt, d_model, ffn, 2200)
    pk = [G.upload(t) for t in tens]
    rng = np.random.default_rng(2201)
    x = rng.standard_normal((n_tok, d_model)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, d_model).astype(np.float32)
    a, _ = _run(fmt, tens, pk, gamma, x, d_model, ffn)
    b, _ = _run(fmt, tens, pk, gamma, x, d_model, ffn, in_place=True)
    assert np.array_equal(a, b)


def test_block_zero_down_is_the_residual():
    d_model, ffn = 288, 768
    rng = np.random.default_rng(2300)
    tg = synth.make_tensor("q4_0", ffn, d_model, rng)
    tu = synth.make_tensor("q4_0", ffn, d_model, rng)
    dd, qd = synth.draw_q4_0(rng, d_model, ffn)
    td = synth.QTensor("down", "q4_0", d_model, ffn, synth.pack_q4_0(np.zeros_like(dd), qd))
    pk = [G.upload(t) for t in (tg, tu, td)]
    for n_tok in (1, 5):
        x = rng.standard_normal((n_tok, d_model)).astype(np.float32)
        gamma = rng.uniform(0.5, 1.5, d_model).astype(np.float32)
        out, _ = _run("q4_0", (tg, tu, td), pk, gamma, x, d_model, ffn)
        assert np.array_equal(out, x)


def test_block_fullsize_27b_sampled():
    # the 27B-class FFN block at 1 token (fused GEMV) and 8 tokens (matrix
    # cores): h and out on sampled rows
    w = synth.CFG5
    tens = synth.gen_workload(w)
    pk = [G.upload(t) for t in tens]
    rng = np.random.default_rng(2400)
    gamma = rng.uniform(0.5, 1.5, w.d_model).astype(np.float32)
    for n_tok in (1, 8):
        x = synth.gen_x(w, w.d_model, n_tok, which=30 + n_tok)
        out, h = _run("q4_0", tens, pk, gamma, x, w.d_model, w.ffn)
        rel = G.rel_for("q4_0", n_tok)
        xn, _ = oracle.rmsnorm(x, gamma, EPS)
        # gate/up over all rows is quick enough in the oracle at this size
        r = {}
        r["g"], r["Sg"] = oracle.gemv_f64x("q4_0", tens[0].raw, xn, w.ffn, w.d_model)
        r["u"], r["Su"] = oracle.gemv_f64x("q4_0", tens[1].raw, xn, w.ffn, w.d_model)
        r["h"] = G.silu64(r["g"]) * r["u"]
        assert np.all(np.abs(h - r["h"]) <= G.h_bound(r, rel + NORM_REL)), f"27B block h n_tok={n_tok}"
        for r0 in (0, w.d_model // 2 - 64, w.d_model - 128):
            yr, S = oracle.gemv("q4_0", tens[2].raw, h, w.d_model, w.ffn, row_begin=r0, row_end=r0 + 128)
            want = x[:, r0:r0 + 128].astype(np.float64) + yr
            bound = rel * S + G.ABS + np.abs(want) * 2.0 ** -24
            assert np.all(np.abs(out[:, r0:r0 + 128] - want) <= bound), f"27B block out n_tok={n_tok} rows {r0}.."


@pytest.mark.parametrize("d_model,ffn", [(2048, 512), (5120, 512), (8192, 256), (8224, 256)])
def test_block_matrix_cores_rmsnorm_widths(d_model, ffn):
    # several tokens on the matrix cores: the RMSNorm launch keeps 2, 6 or 8
    # float4 pieces of x per thread in registers; 8224 columns take the
    # strided fallback
    n_tok = 4
    tens = _tensors("q4_0", d_model, ffn, 2300 + d_model)
    rng = np.random.default_rng(2400 + d_model)
    x = (3.0 * rng.standard_normal((n_tok, d_model))).astype(np.float32)
    gamma = rng.uniform(0.2, 2.0, d_model).astype(np.float32)
    check_block("q4_0", tens, x, gamma, d_model, ffn, f"block q4_0 n_tok={n_tok} d_model={d_model}")


@pytest.mark.parametrize("fmt,n_tok", [("q4_0", 8), ("q4_k", 40), ("i8row", 13)])
def test_block_bf16_copies_bit_identical(fmt, n_tok):
    # large matrices from 8 tokens on: the RMSNorm launch also writes the
    # normalized input rounded to bf16 and the gate/up product h's bf16 copy,
    # when swiglu_ffn_block_scratch_elems' room is given; one float less keeps
    # the fp32 inputs. Same rounding, so out and h are bit-identical; the
    # default scratch is checked against the oracle too.
    d_model, ffn = 4096, 4096
    tens = _tensors(fmt, d_model, ffn, 2400 + n_tok)
    pk = [G.upload(t) for t in tens]
    rng = np.random.default_rng(2401 + n_tok)
    x = (2.0 * rng.standard_normal((n_tok, d_model))).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, d_model).astype(np.float32)
    xd, gd = G.torch.from_numpy(x).to(G.dev()), G.torch.from_numpy(gamma).to(G.dev())
    full = G.qg().swiglu_ffn_block_scratch_elems(fmt, d_model, ffn, n_tok)
    res = []
    for elems in (full, full - 1):
        sc = G.torch.full((elems,), float("nan"), device=G.dev())
        out, h = G.qg().swiglu_ffn_block(fmt, pk[0], pk[1], pk[2], gd, 1e-5, xd, d_model, ffn, h_scratch=sc)
        G.torch.cuda.synchronize()
        res.append((out.cpu().numpy(), h.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    if n_tok <= 13:
        check_block(fmt, tens, x, gamma, d_model, ffn, f"block {fmt} n_tok={n_tok} bf16 copies")
