"""GPU parity of the one-token SwiGLU block whose down product runs in K
halves (qgemv_set_ffn_khalf): the gate/up launch sets out to zero, then each
workgroup of the down product adds the sums of one column half of its rows
into out with an atomic add.

Bars: h within its bound of the oracle's silu(g) * u; out within
2e-5 * sum |w h| + 1e-7 of the oracle's down product of the device's own h;
two runs bit-identical (each output is two additions onto an exact zero, which
commute); an out filled with NaN beforehand is fully overwritten; with the
split off, the same bound (the two forms differ only in summation order).
Shapes: the 27B-class block (544 blocks per row, halves of 272, the built-in
choice), the small Q4_0 block (24 blocks: halves of 12), odd block counts
(25: halves of 13 and 12; 33: 17 and 16), two blocks per row (halves of one),
one block per row (no halves: the split declines, whole rows),
forced row-streaming shapes (rows per row-step, ring depth, row-steps per
workgroup, order, workgroups per CU), and several tokens on the per-token loop.
The FFN block out of place (RMSNorm in, residual out: the first half adds the
residual with its sums) against the oracle's block, bit-identical over runs,
the residual itself when the down scales are 0; in place it keeps whole rows
(equal to the out-of-place block with the split off).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _gpu as G
from tests.test_gpu_block import check_block, _run as block_run

pytestmark = pytest.mark.gpu

SHAPES = [(5120, 17408), (288, 768), (96, 800), (64, 1056), (160, 64), (64, 32)]


def _tensors(d_model, ffn, seed):
    rng = np.random.default_rng(seed)
    tens = [synth.make_tensor("q4_0", ffn, d_model, rng), synth.make_tensor("q4_0", ffn, d_model, rng),
            synth.make_tensor("q4_0", d_model, ffn, rng)]
    x = rng.standard_normal((1, d_model)).astype(np.float32)
    return tens, x


def _run(pk, x, d_model, ffn, n_tok=1):
    """swiglu_ffn into an out filled with NaN; (out, h) on the host."""
    t = G.torch
    xd = t.from_numpy(np.ascontiguousarray(x)).to(G.dev())
    out = t.full((n_tok, d_model), float("nan"), device=G.dev())
    hs = t.empty(G.qg().swiglu_ffn_scratch_elems("q4_0", d_model, ffn, n_tok), device=G.dev())
    G.qg().swiglu_ffn("q4_0", pk[0], pk[1], pk[2], xd, d_model, ffn, out=out, h_scratch=hs)
    t.cuda.synchronize()
    return out.cpu().numpy(), hs[: n_tok * ffn].cpu().numpy().reshape(n_tok, ffn)


def _check(tens, x, out, h, d_model, ffn, what):
    r = oracle.swiglu("q4_0", tens[0].raw, tens[1].raw, tens[2].raw, x, d_model, ffn)
    assert np.all(np.abs(h - r["h"]) <= G.h_bound(r)), f"{what}: h outside its bound"
    yr, S = G.oracle_gemv_rows("q4_0", tens[2].raw, h, d_model, ffn)
    G.check_bound(out, yr, S, what=f"{what} down")


@pytest.mark.parametrize("d_model,ffn", SHAPES)
def test_khalf_ffn_within_bound_and_deterministic(d_model, ffn):
    tens, x = _tensors(d_model, ffn, 7000 + ffn)
    pk = [G.upload(t) for t in tens]
    try:
        G.qg().set_ffn_khalf(0 if ffn >= 8192 else 2)
        out1, h1 = _run(pk, x, d_model, ffn)
        out2, h2 = _run(pk, x, d_model, ffn)
        assert not np.isnan(out1).any()
        assert np.array_equal(out1, out2) and np.array_equal(h1, h2)
        _check(tens, x, out1, h1, d_model, ffn, f"K halves {d_model}/{ffn}")
        G.qg().set_ffn_khalf(1)
        out0, h0 = _run(pk, x, d_model, ffn)
        assert np.array_equal(h0, h1)
        _check(tens, x, out0, h0, d_model, ffn, f"whole rows {d_model}/{ffn}")
    finally:
        G.qg().set_ffn_khalf(0)


@pytest.mark.parametrize("d_model,ffn", [(288, 768), (96, 800), (5120, 17408)])
def test_khalf_forced_shapes(d_model, ffn):
    # the override's fields apply to both products of the block; a combination
    # that one of them does not take runs that product on the lane-group
    # kernel and the block unsplit, which must be correct too
    tens, x = _tensors(d_model, ffn, 7100 + ffn)
    pk = [G.upload(t) for t in tens]
    cfgs = [(rs, 0, depth, nrs, order, wpc)
            for rs in (1, 2, 4) for depth in (2, 4) for nrs in (0, 1, 3) for order in (0, 1) for wpc in (0, 2)]
    if ffn > 5000:
        cfgs = cfgs[::6]
    try:
        G.qg().set_ffn_khalf(2)
        for cfg in cfgs:
            G.qg().set_xs_override(1, *cfg)
            out, h = _run(pk, x, d_model, ffn)
            assert not np.isnan(out).any(), cfg
            _check(tens, x, out, h, d_model, ffn, f"K halves {d_model}/{ffn} cfg {cfg}")
    finally:
        G.qg().set_xs_override(0)
        G.qg().set_ffn_khalf(0)


def test_khalf_per_token_loop():
    # several tokens with the matrix-core path off: every token's gate/up
    # clears its own row of out before any down product adds into it
    d_model, ffn, n_tok = 288, 768, 3
    rng = np.random.default_rng(7200)
    tens = [synth.make_tensor("q4_0", ffn, d_model, rng), synth.make_tensor("q4_0", ffn, d_model, rng),
            synth.make_tensor("q4_0", d_model, ffn, rng)]
    x = rng.standard_normal((n_tok, d_model)).astype(np.float32)
    pk = [G.upload(t) for t in tens]
    try:
        G.qg().set_prefill_override(-1, 0, 0, 0, 0)
        G.qg().set_ffn_khalf(2)
        out, h = _run(pk, x, d_model, ffn, n_tok)
        assert not np.isnan(out).any()
        _check(tens, x, out, h, d_model, ffn, "K halves, 3 tokens")
    finally:
        G.qg().set_prefill_override(0, 0, 0, 0, 0)
        G.qg().set_ffn_khalf(0)


@pytest.mark.parametrize("d_model,ffn", [(5120, 17408), (288, 768), (96, 800)])
def test_khalf_block_out_of_place(d_model, ffn):
    rng = np.random.default_rng(7300 + ffn)
    tens = [synth.make_tensor("q4_0", ffn, d_model, rng), synth.make_tensor("q4_0", ffn, d_model, rng),
            synth.make_tensor("q4_0", d_model, ffn, rng)]
    x = (3.0 * rng.standard_normal((1, d_model))).astype(np.float32)
    gamma = rng.uniform(0.2, 2.0, d_model).astype(np.float32)
    try:
        G.qg().set_ffn_khalf(0 if ffn >= 8192 else 2)
        pk, out1 = check_block("q4_0", tens, x, gamma, d_model, ffn, f"K-halves block {d_model}/{ffn}")
        out2, _ = block_run("q4_0", tens, pk, gamma, x, d_model, ffn)
        assert np.array_equal(out1, out2)
        # in place: whole rows, whatever the switch says
        inp, _ = block_run("q4_0", tens, pk, gamma, x, d_model, ffn, in_place=True)
        G.qg().set_ffn_khalf(1)
        whole, _ = block_run("q4_0", tens, pk, gamma, x, d_model, ffn)
        assert np.array_equal(inp, whole)
    finally:
        G.qg().set_ffn_khalf(0)


def test_khalf_block_zero_down_is_the_residual():
    d_model, ffn = 288, 768
    rng = np.random.default_rng(7400)
    tg = synth.make_tensor("q4_0", ffn, d_model, rng)
    tu = synth.make_tensor("q4_0", ffn, d_model, rng)
    dd, qd = synth.draw_q4_0(rng, d_model, ffn)
    td = synth.QTensor("down", "q4_0", d_model, ffn, synth.pack_q4_0(np.zeros_like(dd), qd))
    pk = [G.upload(t) for t in (tg, tu, td)]
    x = rng.standard_normal((1, d_model)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, d_model).astype(np.float32)
    try:
        G.qg().set_ffn_khalf(2)
        out, _ = block_run("q4_0", (tg, tu, td), pk, gamma, x, d_model, ffn)
        assert np.array_equal(out, x)
    finally:
        G.qg().set_ffn_khalf(0)


def test_khalf_graph_replays():
    # the 27B-class FFN and out-of-place block at one token (gate/up clearing
    # out, down in K halves with atomic adds) captured in one HIP graph and
    # replayed three times, out filled with NaN before each replay and eager
    # calls between them: every replay equals the eager calls bit for bit
    d_model, ffn = 5120, 17408
    torch = G.torch
    tens, x = _tensors(d_model, ffn, 7500)
    pk = [G.upload(t) for t in tens]
    xd = torch.from_numpy(x).to(G.dev())
    gd = torch.from_numpy(np.random.default_rng(7501).uniform(0.5, 1.5, d_model).astype(np.float32)).to(G.dev())
    sf = torch.empty(G.qg().swiglu_ffn_scratch_elems("q4_0", d_model, ffn, 1), device=G.dev())
    sb = torch.empty(G.qg().swiglu_ffn_block_scratch_elems("q4_0", d_model, ffn, 1), device=G.dev())
    of, ob = torch.empty((1, d_model), device=G.dev()), torch.empty((1, d_model), device=G.dev())

    def calls():
        G.qg().swiglu_ffn("q4_0", pk[0], pk[1], pk[2], xd, d_model, ffn, out=of, h_scratch=sf)
        G.qg().swiglu_ffn_block("q4_0", pk[0], pk[1], pk[2], gd, 1e-5, xd, d_model, ffn, out=ob, h_scratch=sb)

    calls()
    torch.cuda.synchronize()
    want_f, want_b = of.clone(), ob.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for k in range(3):
        of.fill_(float("nan"))
        ob.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(of, want_f) and torch.equal(ob, want_b), f"replay {k}"
        G.qg().swiglu_ffn("q4_0", pk[0], pk[1], pk[2], xd, d_model, ffn, out=torch.empty_like(of),
                          h_scratch=torch.empty_like(sf))   # eager work between the replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("d_model,ffn", [(5120, 17408), (288, 768), (96, 800)])
def test_khalf_ffn_q8act(d_model, ffn):
    # the Q8_0-activation FFN at one token with its down product in K halves:
    # each lane quantizes its own chunk of h, so the halves see the blocks the
    # whole rows would; out within the bound of the oracle's product with the
    # device's h quantized, bit-identical over runs, NaN overwritten
    tens, x = _tensors(d_model, ffn, 7600 + ffn)
    pk = [G.upload(t) for t in tens]
    t = G.torch
    xd = t.from_numpy(x).to(G.dev())

    def run():
        out = t.full((1, d_model), float("nan"), device=G.dev())
        o, h = G.qg().swiglu_ffn_q8act("q4_0", pk[0], pk[1], pk[2], xd, d_model, ffn, out=out)
        t.cuda.synchronize()
        return o.cpu().numpy(), h.cpu().numpy()

    try:
        G.qg().set_ffn_khalf(0 if ffn >= 8192 else 2)
        o1, h1 = run()
        o2, h2 = run()
        assert not np.isnan(o1).any()
        assert np.array_equal(o1, o2) and np.array_equal(h1, h2)
        yr, S = oracle.gemv_q8act("q4_0", tens[2].raw, h1, d_model, ffn)
        G.check_bound(o1, yr, S, what=f"q8act K halves {d_model}/{ffn}")
        G.qg().set_ffn_khalf(1)
        o0, h0 = run()
        assert np.array_equal(h0, h1)
        G.check_bound(o0, yr, S, what=f"q8act whole rows {d_model}/{ffn}")
    finally:
        G.qg().set_ffn_khalf(0)
