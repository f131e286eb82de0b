"""GPU parity of the row-streaming one-token kernel (each lane keeps one
block's activations in registers and streams that block of consecutive rows),
which Q4_0 products of one token take by default, under every configuration
the library can launch, and of the lane-group kernels it replaces (still taken
with qgemv_set_xs_override(-1) or any launch override).

Bars as in test_gpu_parity: within 2e-5 * sum |w x| + 1e-7 of the oracle;
bit-identical to it on inputs whose every partial sum is exact (power-of-two
scales, small-integer x), so any summation order must reproduce it; one-hot x
gives the weight column; two runs bit-identical.  Shapes: ragged row counts
(1, 7, 33, 131, ...), rows of 1 to 544 blocks (spare lanes in the last
segment, padded segments), every rows-per-step / depth / row-steps / order
choice, both row orders, the gate/up pair, the normalized gate/up and the
residual down (through swiglu_ffn_block).
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from tests import _gpu as G
from tests.test_gpu_block import check_block

pytestmark = pytest.mark.gpu

SHAPES = [(1, 32), (7, 288), (131, 576), (200, 1536), (97, 5120), (33, 17408), (1000, 2048), (64, 1024)]


def _cfgs(nchunk, nmat):
    """Every forced configuration valid for the shape (the library would run
    an invalid one on the lane-group kernels, which is also correct)."""
    seg0 = (nchunk + 31) // 32
    out = []
    for rs, seg in itertools.product((1, 2, 4, 8), (seg0, seg0 + 1)):
        if (rs * seg) % 2 or rs * seg // 2 > 16 or seg > 32:
            continue
        for d in ((2, 4, 8) if nmat == 1 else (2, 4)):
            for nrs in (1, d, 3 * d + 1):
                for order in (0, 1):
                    out.append((rs, seg, d, nrs, order, 0))
        out.append((rs, seg, (2, 4, 8)[rs % 3] if nmat == 1 else 2, 0, 1, 1 + rs % 3))   # whole workgroups per CU
    return out


def _pow2_q4_0(rows, cols, rng):
    d = (2.0 ** rng.integers(-6, -2, (rows, cols // 32))).astype(np.float16)
    return synth.QTensor("w", "q4_0", rows, cols, synth.pack_q4_0(d, rng.integers(0, 16, (rows, cols))))


def _set(cfg):
    G.qg().set_xs_override(1, *cfg)


def _reset():
    G.qg().set_xs_override(0)


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_xs_exact_inputs_bit_exact_every_config(rows, cols):
    rng = np.random.default_rng(rows * 31 + cols)
    t = _pow2_q4_0(rows, cols, rng)
    pk = G.upload(t)
    x = rng.integers(-2, 3, cols).astype(np.float32)
    yr, _ = oracle.gemv("q4_0", t.raw, x, rows, cols)
    cfgs = [None] + _cfgs(cols // 32, 1)
    try:
        for cfg in cfgs:
            if cfg is None:
                _reset()
            else:
                _set(cfg)
            y = G.gemv_gpu(t, pk, x)
            assert np.array_equal(y.astype(np.float64), yr), f"{rows}x{cols} cfg {cfg}"
    finally:
        _reset()


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_xs_within_bound_and_legacy(rows, cols):
    rng = np.random.default_rng(rows * 17 + cols + 1)
    t = synth.make_tensor("q4_0", rows, cols, rng)
    pk = G.upload(t)
    x = rng.standard_normal(cols).astype(np.float32)
    yr, S = oracle.gemv("q4_0", t.raw, x, rows, cols)
    try:
        for mode in (0, -1):
            G.qg().set_xs_override(mode)
            y1 = G.gemv_gpu(t, pk, x)
            y2 = G.gemv_gpu(t, pk, x)
            assert np.array_equal(y1, y2)
            G.check_bound(y1, yr, S, what=f"{rows}x{cols} mode {mode}")
        for cfg in _cfgs(cols // 32, 1)[::5]:
            _set(cfg)
            G.check_bound(G.gemv_gpu(t, pk, x), yr, S, what=f"{rows}x{cols} cfg {cfg}")
    finally:
        _reset()


def test_xs_one_hot_every_block_position():
    rows, cols = 131, 5120
    t = synth.make_tensor("q4_0", rows, cols, np.random.default_rng(4100))
    pk = G.upload(t)
    w32 = oracle.dequant("q4_0", t.raw, rows, cols)
    nb = cols // 32
    cs = [32 * (k % nb) + k % 32 for k in range(0, 5 * 32, 5)] + [cols - 1]
    for c in cs:
        x = np.zeros(cols, np.float32)
        x[c] = 1.0
        assert np.array_equal(G.gemv_gpu(t, pk, x), w32[:, c]), c


@pytest.mark.parametrize("ffn,d_model", [(17408, 5120), (131, 576), (300, 288), (1000, 2048)])
def test_xs_gate_up_pair_every_config(ffn, d_model):
    # h = silu(Wg x) * (Wu x) on integer inputs: g and u exact, so h equals
    # silu applied to the oracle's exact g and u within the device silu budget
    rng = np.random.default_rng(ffn + d_model)
    tg, tu = _pow2_q4_0(ffn, d_model, rng), _pow2_q4_0(ffn, d_model, rng)
    pg, pu = G.upload(tg), G.upload(tu)
    x = rng.integers(-2, 3, d_model).astype(np.float32)
    g, _ = oracle.gemv("q4_0", tg.raw, x, ffn, d_model)
    u, _ = oracle.gemv("q4_0", tu.raw, x, ffn, d_model)
    want = G.silu64(g) * u
    xd = G.torch.from_numpy(x).to(G.dev())
    cfgs = [None] + _cfgs(d_model // 32, 2)
    if ffn > 5000:
        cfgs = cfgs[::4]
    try:
        for cfg in cfgs:
            if cfg is None:
                _reset()
            else:
                _set(cfg)
            h = G.qg().swiglu_gate_up("q4_0", pg, pu, xd, d_model, ffn)
            G.torch.cuda.synchronize()
            h = h.cpu().numpy().reshape(-1).astype(np.float64)
            assert np.all(np.abs(h - want) <= G.SILU_REL * np.abs(want) + 1e-30), f"cfg {cfg}"
    finally:
        _reset()


@pytest.mark.parametrize("d_model,ffn", [(5120, 17408), (576, 1536), (288, 768)])
def test_xs_block_norm_and_residual(d_model, ffn):
    # swiglu_ffn_block at one token: the normalized gate/up pair and the
    # residual down both on the row-streaming kernel, against the oracle
    rng = np.random.default_rng(4200 + d_model)
    tens = [synth.make_tensor("q4_0", ffn, d_model, rng), synth.make_tensor("q4_0", ffn, d_model, rng),
            synth.make_tensor("q4_0", d_model, ffn, rng)]
    x = rng.standard_normal((1, d_model)).astype(np.float32)
    gamma = (rng.random(d_model) + 0.5).astype(np.float32)
    check_block("q4_0", tens, x, gamma, d_model, ffn, f"xs block {d_model}/{ffn}")
