"""GPU parity of greedy sampling (qgemv_argmax, qgemv_head_argmax) through the C ABI.

Bars:
  * qgemv_argmax on given logits: the same index as the oracle's in-order scan,
    bit for bit (integer output), over crafted rows -- planted ties with the
    maximum, infinities, signed zeros, NaN anywhere and at index 0 -- and sizes
    around the 64-lane and 256-thread boundaries up to vocabulary widths;
  * qgemv_head_argmax: the token is the oracle argmax of the device's own
    logits (unique), and it is a valid argmax of the exact logits: its exact
    logit is within the two logits' error bounds of the exact maximum.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _gpu_argmax(v):
    vd = G.torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(G.dev())
    t = G.qg().qgemv_argmax(vd, v.shape[-1])
    G.torch.cuda.synchronize()
    return t.cpu().numpy()


# sizes for every per-thread piece count of the one-round kernel (1, 2, 4, 6-8, 9-12, 13-16 pieces of
# 4 floats per thread), the unaligned path (n % 4 != 0) and the multi-round path (> 65536)
@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 255, 256, 257, 1000, 4097, 4100, 8192, 12000, 32000, 40000,
                               49152, 65536, 65540, 151936])
def test_argmax_random_rows_with_ties(n):
    rng = np.random.default_rng(n)
    v = rng.standard_normal((5, n)).astype(np.float32)
    for t in range(5):   # plant copies of the maximum (ties) at random places
        k = rng.integers(1, 4)
        v[t, rng.integers(0, n, k)] = v[t].max() + (t % 2)
    got = _gpu_argmax(v)
    assert [int(a) for a in got] == [oracle.argmax(row) for row in v]


@pytest.mark.parametrize("n", [3000, 40000, 65536])
def test_argmax_special_values(n):
    inf, nan = np.inf, np.nan
    rows = [
        [1.0, 3.0, 3.0, 2.0], [-inf, -inf, -inf, -inf], [-inf, -3e38, -inf, -inf], [1.0, inf, inf, 0.0],
        [-0.0, 0.0, -0.0, 0.0], [5.0, nan, 7.0, nan], [nan, 5.0, 9.0, 1.0], [2.0, nan, nan, nan],
        [nan, nan, nan, nan], [-1.0, -0.5, -0.5, -2.0],
    ]
    v = np.array(rows, np.float32)
    assert [int(a) for a in _gpu_argmax(v)] == [oracle.argmax(r) for r in v]
    # the same patterns spread over a long row: specials in different lanes, waves and pieces
    rng = np.random.default_rng(7)
    long = rng.uniform(-1, 1, (6, n)).astype(np.float32)
    long[0, [17, 1200, n - 1]] = 5.0                      # three-way tie
    long[1, ::7] = np.nan                                   # NaNs everywhere except index 0
    long[2, 0] = np.nan                                     # NaN at index 0
    long[3, [100, 900]] = np.inf
    long[4, :] = -np.inf
    long[4, 2500] = -1e30
    long[5, :] = 0.0
    long[5, ::3] = -0.0
    assert [int(a) for a in _gpu_argmax(long)] == [oracle.argmax(r) for r in long]


def _check_head(t, n_tok, seed):
    pk = G.upload(t)
    x = np.random.default_rng(seed).standard_normal((n_tok, t.cols)).astype(np.float32)
    xd = G.torch.from_numpy(x).to(G.dev())
    tok, logits = G.qg().qgemv_head_argmax(t.fmt, pk, xd, t.rows, t.cols, fused=True)
    G.torch.cuda.synchronize()
    tok, logits = tok.cpu().numpy(), logits.cpu().numpy()
    tok2, logits2 = G.qg().qgemv_head_argmax(t.fmt, pk, xd, t.rows, t.cols)
    G.torch.cuda.synchronize()
    assert np.array_equal(tok, tok2.cpu().numpy()) and np.array_equal(logits, logits2.cpu().numpy())
    yr, S = oracle.gemv(t.fmt, t.raw, x, t.rows, t.cols, row_scale=t.row_scale)
    rel = G.rel_for(t.fmt, n_tok)
    for k in range(n_tok):
        assert int(tok[k]) == oracle.argmax(logits[k])
        b = rel * S[k] + G.ABS
        m = int(np.argmax(yr[k]))
        assert yr[k][tok[k]] >= yr[k][m] - (b[tok[k]] + b[m]), f"token {k}: not a valid argmax of the exact logits"


@pytest.mark.parametrize("wname,idx,n_tok", [(synth.CFG2.name, 7, 1), (synth.CFG2.name, 7, 3),
                                             (synth.CFG4.name, 3, 1)])
def test_head_argmax_vocab_heads(wname, idx, n_tok):
    # the SmolLM2-135M Q8_0 head and the SmolLM2-1.7B INT8-row head, 49152 rows
    w = synth.WORKLOADS[wname]
    t = synth.gen_tensor(w, idx)
    assert t.rows == 49152
    _check_head(t, n_tok, 40 + n_tok)


def test_head_argmax_q6_k_head():
    # TinyLlama's Q6_K vocab head, 32000 rows
    t = synth.gen_tensor(synth.CFG6, 1)
    assert (t.fmt, t.rows) == ("q6_k", 32000)
    _check_head(t, 1, 47)


def test_head_argmax_matrix_cores():
    # a Q4_0 head at 8 tokens runs the product on the matrix cores first
    t = synth.make_tensor("q4_0", 4096, 1024, np.random.default_rng(45))
    _check_head(t, 8, 46)


# ------------------------------------------------------------ fused head --
# qgemv_head_argmax_ws at one token: the argmax fused into the product's
# epilogue (one candidate per workgroup), then a one-workgroup launch that
# combines the candidates. Bars: the logits bit-identical to the two-launch
# path's (the same product kernel), the token identical to its token and to
# the oracle argmax of the device logits; one workspace reused call after
# call across shapes, starting from garbage (no initialization needed) and
# holding the number of candidates of the last call; ties, NaN at index 0
# and NaN elsewhere by the in-order rule.

FUSED_SHAPES = {"q4_0": [(1, 64), (7, 288), (131, 576), (4099, 2048), (40000, 576)],
                "q8_0": [(1, 32), (7, 288), (131, 576), (4099, 2048), (40000, 576)],
                "i8row": [(1, 32), (7, 288), (131, 576), (4099, 2048)],
                "q4_k": [(1, 256), (7, 512), (131, 768), (4099, 2048)],
                "q6_k": [(1, 256), (7, 512), (131, 768), (4099, 2048)]}


def _head(t, pk, x, fused, ws=None):
    xd = G.torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(G.dev())
    tok, logits = G.qg().qgemv_head_argmax(t.fmt, pk, xd, t.rows, t.cols, workspace=ws, fused=fused)
    G.torch.cuda.synchronize()
    return int(tok.cpu().numpy()[0]), logits.cpu().numpy().reshape(-1)


@pytest.mark.parametrize("fmt,rows,cols", [(f, r, c) for f, sh in FUSED_SHAPES.items() for r, c in sh])
def test_fused_head_matches_two_launches(fmt, rows, cols):
    rng = np.random.default_rng(rows + cols + len(fmt))
    t = synth.make_tensor(fmt, rows, cols, rng)
    pk = G.upload(t)
    x = rng.standard_normal(cols).astype(np.float32)
    modes = [0, -1] if fmt == "q4_0" else [0]     # Q4_0: the row-streaming and the lane-group kernels
    try:
        for mode in modes:
            G.qg().set_xs_override(mode)
            tf, lf = _head(t, pk, x, True)
            t2, l2 = _head(t, pk, x, False)
            assert np.array_equal(lf, l2), f"mode {mode}: fused logits differ"
            assert tf == t2 == oracle.argmax(lf), f"mode {mode}: token {tf} vs {t2}"
    finally:
        G.qg().set_xs_override(0)


def test_fused_head_workspace_reused():
    # one workspace through calls of several shapes and inputs, filled with
    # 0xFF bytes first: each token right, the header holding a candidate
    # count within the workspace after every call
    rng = np.random.default_rng(4700)
    heads = [synth.make_tensor("q8_0", r, c, rng) for r, c in ((40000, 576), (300, 288), (4099, 2048))]
    heads.append(synth.make_tensor("q4_0", 20000, 1024, rng))
    pks = [G.upload(t) for t in heads]
    need = max(G.qg().head_argmax_workspace_bytes(t.fmt, t.rows, t.cols) for t in heads)
    ws = G.torch.full((need,), 255, dtype=G.torch.uint8, device=G.dev())
    for k in range(12):
        t, pk = heads[k % 4], pks[k % 4]
        x = rng.standard_normal(t.cols).astype(np.float32)
        tok, logits = _head(t, pk, x, True, ws)
        assert tok == oracle.argmax(logits), k
        n = int(ws[:4].cpu().numpy().view(np.uint32)[0])
        assert 1 <= n <= min(t.rows, (need - 256) // 8), f"call {k}: {n} candidates"


def _q8_0_rows(d_rows, codes):
    """A Q8_0 tensor with per-row constant f16 scales (given as uint16 bits) and given codes."""
    rows, cols = codes.shape
    d = np.repeat(np.asarray(d_rows, np.uint16)[:, None], cols // 32, axis=1).view(np.float16)
    return synth.QTensor("w", "q8_0", rows, cols, synth.pack_q8_0(d, codes.astype(np.int8)))


@pytest.mark.parametrize("rows", [300, 40000])
def test_fused_head_ties_and_nan(rows):
    cols = 64
    x = np.ones(cols, np.float32)
    one, two, inf = 0x3C00, 0x4000, 0x7C00      # f16 1.0, 2.0, +inf
    codes = np.full((rows, cols), 3, np.int64)
    base = np.full(rows, one, np.uint16)
    cases = []
    # tie: two rows far apart share the largest logit -> the first of them
    d = base.copy(); d[[rows // 3, rows - 2]] = two
    cases.append((d, codes.copy()))
    # NaN at row 0 (scale inf times code 0) -> 0, whatever the largest is
    d = base.copy(); d[0] = inf; c = codes.copy(); c[0] = 0; d[rows // 2] = two
    cases.append((d, c))
    # NaN in the middle, the maximum after it -> the maximum
    d = base.copy(); d[5] = inf; c = codes.copy(); c[5] = 0; d[rows - 1] = two
    cases.append((d, c))
    # every logit equal -> 0
    cases.append((base.copy(), codes.copy()))
    for k, (d, c) in enumerate(cases):
        t = _q8_0_rows(d, c)
        pk = G.upload(t)
        tok, logits = _head(t, pk, x, True)
        assert tok == oracle.argmax(logits), (k, tok)
        assert tok == [rows // 3, 0, rows - 1, 0][k], (k, tok)
