"""Full-size parity: every matrix of the five workloads at its real shape, in
the launch configuration the library picks for it (the one bench.py times),
against the CPU oracle on every output element (the scalar oracle streams
these sizes in about a second each).

Workloads (seeded synthetic inputs, synth.WORKLOADS): the Q4_0 SwiGLU FFN of a
stories15M-sized model (288/768); a SmolLM2-135M-shaped decode layer in Q4_0
with its Q8_0 vocab head (576 -> 49152); a TinyLlama-1.1B-shaped layer in Q4_K;
a SmolLM2-1.7B-shaped per-row INT8 FFN and head (2048 -> 49152); a 27B-class
Q4_0 FFN (5120/17408).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _gemv_cases():
    out = []
    for w in synth.WORKLOADS.values():
        for i, (name, fmt, rows, cols) in enumerate(w.tensors):
            out.append(pytest.param(w.name, i, id=f"cfg{w.cfg_id}-{name}"))
    return out


@pytest.mark.parametrize("wname,idx", _gemv_cases())
def test_fullsize_gemv(wname, idx):
    w = synth.WORKLOADS[wname]
    t = synth.gen_tensor(w, idx)
    x = synth.gen_x(w, t.cols, 1, which=idx)
    y = G.gemv_gpu(t, G.upload(t), x[0])
    yr, S = oracle.gemv(t.fmt, t.raw, x[0], t.rows, t.cols, row_scale=t.row_scale)
    G.check_bound(y, yr, S, what=f"{wname} {t.name} {t.rows}x{t.cols}")


@pytest.mark.parametrize("wname", [synth.CFG1.name, synth.CFG5.name])
def test_fullsize_swiglu_ffn(wname):
    w = synth.WORKLOADS[wname]
    tens = synth.gen_workload(w)
    x = synth.gen_x(w, w.d_model, 1)
    pk = [G.upload(t) for t in tens]
    xd = G.torch.from_numpy(x).to(G.dev())
    out, h = G.qg().swiglu_ffn(tens[0].fmt, pk[0], pk[1], pk[2], xd, w.d_model, w.ffn)
    G.torch.cuda.synchronize()
    out = out.cpu().numpy()
    h = h.cpu().numpy()
    r = {}
    r["g"], r["Sg"] = oracle.gemv(tens[0].fmt, tens[0].raw, x, w.ffn, w.d_model)
    r["u"], r["Su"] = oracle.gemv(tens[1].fmt, tens[1].raw, x, w.ffn, w.d_model)
    r["h"] = G.silu64(r["g"]) * r["u"]
    assert np.all(np.abs(h - r["h"]) <= G.h_bound(r)), "h outside its bound"
    yr, S = oracle.gemv(tens[2].fmt, tens[2].raw, h, w.d_model, w.ffn)
    G.check_bound(out, yr, S, what=f"{wname} down")


@pytest.mark.parametrize("wname,ffn_idx", [(synth.CFG2.name, (4, 5, 6)), (synth.CFG3.name, (3, 4, 5)),
                                           (synth.CFG4.name, (0, 1, 2))])
def test_fullsize_swiglu_other_formats(wname, ffn_idx):
    # the FFN matrices of the SmolLM2-135M (Q4_0), TinyLlama (Q4_K) and
    # SmolLM2-1.7B (INT8 row) layers, chained through swiglu_ffn
    w = synth.WORKLOADS[wname]
    tg, tu, td = (synth.gen_tensor(w, i) for i in ffn_idx)
    d_model, ffn = tg.cols, tg.rows
    x = synth.gen_x(w, d_model, 1, which=len(w.tensors))
    pk = [G.upload(t) for t in (tg, tu, td)]
    xd = G.torch.from_numpy(x).to(G.dev())
    out, h = G.qg().swiglu_ffn(tg.fmt, pk[0], pk[1], pk[2], xd, d_model, ffn)
    G.torch.cuda.synchronize()
    out, h = out.cpu().numpy(), h.cpu().numpy()
    r = {}
    r["g"], r["Sg"] = oracle.gemv(tg.fmt, tg.raw, x, ffn, d_model, row_scale=tg.row_scale)
    r["u"], r["Su"] = oracle.gemv(tu.fmt, tu.raw, x, ffn, d_model, row_scale=tu.row_scale)
    r["h"] = G.silu64(r["g"]) * r["u"]
    assert np.all(np.abs(h - r["h"]) <= G.h_bound(r)), "h outside its bound"
    yr, S = oracle.gemv(td.fmt, td.raw, h, d_model, ffn, row_scale=td.row_scale)
    G.check_bound(out, yr, S, what=f"{wname} down")


def test_fullsize_cfg5_batched_tokens_every_row():
    # n_tok = 8 and 128 on the 27B-class gate matrix (matrix-core path), every
    # output element against the oracle
    w = synth.CFG5
    t = synth.gen_tensor(w, 0)
    pk = G.upload(t)
    for n in (8, 128):
        x = synth.gen_x(w, w.d_model, n, which=10 + n)
        y = G.gemv_gpu(t, pk, x)
        yr, S = G.oracle_gemv_rows(t.fmt, t.raw, x, t.rows, t.cols)
        G.check_bound(y, yr, S, rel=G.PF_REL, what=f"cfg5 gate n_tok={n}")


def _check_ffn_every_row(fmt, tens, x, d_model, ffn, what):
    # swiglu_ffn with the scratch swiglu_ffn_scratch_elems asks for (as
    # bench.py runs it): every element of h against silu(g) u of the oracle,
    # every element of out against the oracle's down projection of the
    # device's own h (all of h is an input there)
    g, u, d = tens
    pk = [G.upload(t) for t in (g, u, d)]
    xd = G.torch.from_numpy(np.ascontiguousarray(x)).to(G.dev())
    out, h = G.qg().swiglu_ffn(fmt, pk[0], pk[1], pk[2], xd, d_model, ffn)
    G.torch.cuda.synchronize()
    out, h = out.cpu().numpy(), h.cpu().numpy()
    r = {}
    r["g"], r["Sg"] = G.oracle_gemv_rows(g.fmt, g.raw, x, ffn, d_model, row_scale=g.row_scale)
    r["u"], r["Su"] = G.oracle_gemv_rows(u.fmt, u.raw, x, ffn, d_model, row_scale=u.row_scale)
    r["h"] = G.silu64(r["g"]) * r["u"]
    bad = ~(np.abs(h - r["h"]) <= G.h_bound(r, G.PF_REL))
    assert not bad.any(), f"{what}: {int(bad.sum())} elements of h outside the bound"
    yr, S = G.oracle_gemv_rows(d.fmt, d.raw, h, d_model, ffn, row_scale=d.row_scale)
    G.check_bound(out, yr, S, rel=G.PF_REL, what=f"{what} down")


@pytest.mark.parametrize("n_tok", [8, 128])
def test_fullsize_cfg5_ffn_batched_every_row(n_tok):
    # the whole 27B-class FFN at n_tok = 8 and 128 through swiglu_ffn, in the
    # launch configuration bench.py times
    w = synth.CFG5
    tens = synth.gen_workload(w)
    x = synth.gen_x(w, w.d_model, n_tok, which=20 + n_tok)
    _check_ffn_every_row(tens[0].fmt, tens, x, w.d_model, w.ffn, f"cfg5 n_tok={n_tok}")


@pytest.mark.parametrize("idx", [0, 1])
def test_fullsize_cfg6_q6_k_batched_every_row(idx):
    # the TinyLlama-shaped Q6_K down [2048][5632] and vocab head [32000][2048]
    # at n_tok = 8 and 128 (matrix-core path), every element against the oracle
    w = synth.CFG6
    t = synth.gen_tensor(w, idx)
    pk = G.upload(t)
    for n in (8, 128):
        x = synth.gen_x(w, t.cols, n, which=30 + n + idx)
        y = G.gemv_gpu(t, pk, x)
        yr, S = G.oracle_gemv_rows(t.fmt, t.raw, x, t.rows, t.cols)
        G.check_bound(y, yr, S, rel=G.PF_REL, what=f"cfg6 {t.name} n_tok={n}")


def _ffn_of(tens):
    names = [t.name for t in tens]
    return [tens[names.index(n)] for n in ("gate", "up", "down")]


def test_fullsize_cfg4_int8_ffn_head_128_tokens_every_row():
    # the SmolLM2-1.7B-shaped INT8 FFN (2048/8192) and vocab head [49152][2048]
    # at 128 tokens on the matrix cores, as bench.py times them
    w = synth.CFG4
    tens = synth.gen_workload(w)
    x = synth.gen_x(w, w.d_model, 128, which=40)
    _check_ffn_every_row("i8row", _ffn_of(tens), x, w.d_model, w.ffn, "cfg4 n_tok=128")
    t = tens[[t.name for t in tens].index("head")]
    y = G.gemv_gpu(t, G.upload(t), x)
    yr, S = G.oracle_gemv_rows(t.fmt, t.raw, x, t.rows, t.cols, row_scale=t.row_scale)
    G.check_bound(y, yr, S, rel=G.PF_REL, what="cfg4 head n_tok=128")


def test_fullsize_cfg2_layer_q8_0_head_128_tokens_every_row():
    # the SmolLM2-135M-shaped Q4_0 layer (q, o, k, v, FFN) and its Q8_0 vocab
    # head [49152][576] at 128 tokens on the matrix cores, as bench.py times
    # them, every element against the oracle
    w = synth.CFG2
    tens = synth.gen_workload(w)
    x = synth.gen_x(w, w.d_model, 128, which=41)
    _check_ffn_every_row("q4_0", _ffn_of(tens), x, w.d_model, w.ffn, "cfg2 n_tok=128")
    for t in tens:
        if t.name in ("gate", "up", "down"):
            continue
        y = G.gemv_gpu(t, G.upload(t), x)
        yr, S = G.oracle_gemv_rows(t.fmt, t.raw, x, t.rows, t.cols)
        G.check_bound(y, yr, S, rel=G.PF_REL, what=f"cfg2 {t.name} n_tok=128")
