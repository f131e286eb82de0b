"""Edge cases through the C ABI on the GPU: the widest rows the library takes
(the staged activation row fills the workgroup's LDS), the refusals with real
device buffers (nothing enqueued: the output keeps its contents), zero inputs,
and the smallest shapes."""
import numpy as np
import pytest

import oracle
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu

FMTS = ["q4_0", "q8_0", "q4_k", "i8row", "q6_k"]


@pytest.mark.parametrize("fmt", FMTS)
def test_widest_rows(fmt):
    # cols = qgemv_max_cols(): the largest row whose staged x fits one
    # workgroup's LDS; one block more is refused
    mc = G.qg().max_cols()
    assert mc % 256 == 0 and mc >= 17408
    rows = 40
    rng = np.random.default_rng(5000)
    t = synth.make_tensor(fmt, rows, mc, rng)
    pk = G.upload(t)
    x = rng.standard_normal(mc).astype(np.float32)
    y = G.gemv_gpu(t, pk, x)
    yr, S = oracle.gemv(fmt, t.raw, x, rows, mc, row_scale=t.row_scale)
    G.check_bound(y, yr, S, what=f"{fmt} 40x{mc}")
    xd = G.torch.zeros(mc + 256, device=G.dev())
    yd = G.torch.zeros(rows, device=G.dev())
    st = G.qg().lib.qgemv(G.qg().FORMATS[fmt], G.qg()._ptr(pk), xd.data_ptr(), yd.data_ptr(), rows, mc + 256, 1,
                          None)
    assert st == -2


def test_widest_rows_batched_and_normalized():
    # the matrix-core path and the normalized gate/up at the widest row
    mc = G.qg().max_cols()
    rng = np.random.default_rng(5100)
    t = synth.make_tensor("q4_0", 48, mc, rng)
    pk = G.upload(t)
    x = rng.standard_normal((5, mc)).astype(np.float32)
    y = G.gemv_gpu(t, pk, x)
    yr, S = oracle.gemv("q4_0", t.raw, x, 48, mc)
    G.check_bound(y, yr, S, rel=G.PF_REL, what=f"q4_0 n_tok=5 48x{mc}")
    # gate/up with RMSNorm in, at d_model = max cols (one token)
    d_model, ffn = mc, 64
    tens = [synth.make_tensor("q4_0", ffn, d_model, rng), synth.make_tensor("q4_0", ffn, d_model, rng),
            synth.make_tensor("q4_0", d_model, ffn, rng)]
    pks = [G.upload(tt) for tt in tens]
    x1 = rng.standard_normal((1, d_model)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, d_model).astype(np.float32)
    xd, gd = G.torch.from_numpy(x1).to(G.dev()), G.torch.from_numpy(gamma).to(G.dev())
    out, h = G.qg().swiglu_ffn_block("q4_0", pks[0], pks[1], pks[2], gd, 1e-5, xd, d_model, ffn)
    G.torch.cuda.synchronize()
    r = oracle.ffn_block("q4_0", tens[0].raw, tens[1].raw, tens[2].raw, gamma, 1e-5, x1, d_model, ffn)
    rel = 2e-5 + 4e-6
    Bg, Bu = rel * r["Sg"] + G.ABS, rel * r["Su"] + G.ABS
    sig = 1.0 / (1.0 + np.exp(-r["g"]))
    hb = np.abs(sig * (1 + r["g"] * (1 - sig)) * r["u"]) * Bg + np.abs(r["g"] * sig) * Bu + G.SILU_REL * np.abs(r["h"])
    assert np.all(np.abs(h.cpu().numpy() - r["h"]) <= hb + 1e-30)


@pytest.mark.parametrize("fmt", FMTS)
def test_widest_rows_batched_every_format(fmt):
    # the matrix-core path at the widest row the GEMV takes (the matrix-core
    # kernel streams K, so its LDS does not grow with cols): ragged rows,
    # a partial token tile
    mc = G.qg().max_cols()
    rng = np.random.default_rng(5150)
    t = synth.make_tensor(fmt, 37, mc, rng)
    x = rng.standard_normal((5, mc)).astype(np.float32)
    y = G.gemv_gpu(t, G.upload(t), x)
    yr, S = oracle.gemv(fmt, t.raw, x, 37, mc, row_scale=t.row_scale)
    G.check_bound(y, yr, S, rel=G.PF_REL, what=f"{fmt} n_tok=5 37x{mc}")


def _bufs(rows, cols, n_tok=1):
    t = synth.make_tensor("q4_0", rows, cols, np.random.default_rng(5200))
    pk = G.upload(t)
    x = G.torch.randn(n_tok * cols + 64, device=G.dev())
    y = G.torch.full((n_tok * rows + 64,), 7.0, device=G.dev())
    return t, pk, x, y


def test_refusals_enqueue_nothing():
    # each refused call returns its status and leaves y untouched
    lib, P = G.qg().lib, G.qg()._ptr
    rows, cols = 64, 512
    t, pk, x, y = _bufs(rows, cols)
    xp, yp = x.data_ptr(), y.data_ptr()
    cases = {
        "unknown format": (lib.qgemv(9, P(pk), xp, yp, rows, cols, 1, None), -4),
        "null packed": (lib.qgemv(0, None, xp, yp, rows, cols, 1, None), -1),
        "no rows": (lib.qgemv(0, P(pk), xp, yp, 0, cols, 1, None), -2),
        "no tokens": (lib.qgemv(0, P(pk), xp, yp, rows, cols, 0, None), -2),
        "ragged cols": (lib.qgemv(0, P(pk), xp, yp, rows, cols - 16, 1, None), -2),
        "misaligned x": (lib.qgemv(0, P(pk), xp + 4, yp, rows, cols, 1, None), -3),
        "misaligned packed": (lib.qgemv(0, P(pk) + 16, xp, yp, rows, cols, 1, None), -3),
        "x overlaps y": (lib.qgemv(0, P(pk), yp, yp + 64, rows, cols, 1, None), -5),
        "y inside packed": (lib.qgemv(0, P(pk), xp, P(pk) + 256, rows, cols, 1, None), -5),
    }
    G.torch.cuda.synchronize()
    for what, (st, want) in cases.items():
        assert st == want, (what, st)
    assert G.torch.all(y == 7.0)


def test_ffn_refusals_enqueue_nothing():
    lib, P = G.qg().lib, G.qg()._ptr
    d_model, ffn = 256, 512
    rng = np.random.default_rng(5300)
    tens = [synth.make_tensor("q4_0", ffn, d_model, rng), synth.make_tensor("q4_0", ffn, d_model, rng),
            synth.make_tensor("q4_0", d_model, ffn, rng)]
    pk = [G.upload(tt) for tt in tens]
    x = G.torch.randn(d_model, device=G.dev())
    out = G.torch.full((d_model,), 7.0, device=G.dev())
    h = G.torch.full((ffn,), 7.0, device=G.dev())
    a = [P(p) for p in pk]
    assert lib.swiglu_ffn(0, *a, x.data_ptr(), out.data_ptr(), h.data_ptr(), ffn - 1, d_model, ffn, 1, None) == -6
    assert lib.swiglu_ffn(0, *a, x.data_ptr(), out.data_ptr(), out.data_ptr(), ffn, d_model, ffn, 1, None) == -5
    assert lib.swiglu_ffn_q8act(2, *a, x.data_ptr(), out.data_ptr(), h.data_ptr(), ffn, d_model, ffn, 1, None) == -4
    G.torch.cuda.synchronize()
    assert G.torch.all(out == 7.0) and G.torch.all(h == 7.0)


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_activations_give_zero(fmt):
    rows, cols = 70, 2048
    t = synth.make_tensor(fmt, rows, cols, np.random.default_rng(5400))
    pk = G.upload(t)
    y = G.gemv_gpu(t, pk, np.zeros(cols, np.float32))
    assert np.all(y == 0)
    if fmt in ("q4_0", "q8_0"):
        y8 = G.qg().qgemv_q8act(fmt, pk, G.torch.zeros(cols, device=G.dev()), rows, cols)
        G.torch.cuda.synchronize()
        assert G.torch.all(y8 == 0)


@pytest.mark.parametrize("fmt,cols", [("q4_0", 32), ("q8_0", 32), ("i8row", 32), ("q4_k", 256), ("q6_k", 256)])
def test_single_row_single_block(fmt, cols):
    rng = np.random.default_rng(5500)
    t = synth.make_tensor(fmt, 1, cols, rng)
    pk = G.upload(t)
    for n_tok in (1, 2, 17):
        x = rng.standard_normal((n_tok, cols)).astype(np.float32)
        y = G.gemv_gpu(t, pk, x)
        yr, S = oracle.gemv(fmt, t.raw, x, 1, cols, row_scale=t.row_scale)
        G.check_bound(y, yr, S, rel=G.rel_for(fmt, n_tok), what=f"{fmt} 1x{cols} n_tok={n_tok}")
