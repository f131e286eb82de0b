"""GPU parity of the Q8_0-activation mode (the Go "llm" package's ExactGGML:
activations quantised to Q8_0 before each quantised product) through the C ABI.

Bars:
  * the quantized activation blocks (binary16 scale and the 32 codes) are
    byte-identical to the oracle's: the same decisions in the same binary32
    precision, ties included;
  * y: |y_gpu - y_ref| <= 2e-5 * sum_j |w_ij xq_j| + 1e-7, y_ref the oracle's
    binary64 product with the quantized activations xq (the block products are
    exact integers on the device; only the per-block scaling and the fp32
    accumulation round);
  * weights with power-of-two scales and activations on the Q8_0 grid: every
    partial sum is exact, so y is bit-identical to the oracle;
  * the FFN stage by stage: h against silu(g) u of the oracle's products, out
    against the oracle's down product of the device's own h (quantized again);
  * Q4_0 at one token on the row-streaming kernel (each lane quantizes its own
    chunk of x): the exact-input identity under every launch shape it takes.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu

FMTS = ["q4_0", "q8_0"]


def _oracle_blocks(x, n):
    d, q = oracle.quantize_q8_0(x.reshape(-1, n))
    nb = n // 32
    out = np.empty((d.shape[0], nb, 34), np.uint8)
    out[:, :, 0:2] = d.astype("<u2").view(np.uint8).reshape(d.shape[0], nb, 2)
    out[:, :, 2:] = q.view(np.uint8).reshape(d.shape[0], nb, 32)
    return out.reshape(d.shape[0], nb * 34)


def _gpu_blocks(x, n):
    xd = G.torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(G.dev())
    b = G.qg().qquantize_q8_0(xd, n)
    G.torch.cuda.synchronize()
    return b.cpu().numpy()


def test_quantize_matches_oracle_bytes():
    rng = np.random.default_rng(3000)
    for n, n_tok in ((32, 1), (576, 3), (5120, 2), (17408, 1)):
        x = (rng.standard_normal((n_tok, n)) * 2.0 ** rng.integers(-14, 14, (n_tok, n // 32)).repeat(32, 1))
        x = x.astype(np.float32)
        x[:, 64:96] = 0.0 if n > 96 else x[:, 64:96]                       # a zero block
        assert np.array_equal(_gpu_blocks(x, n), _oracle_blocks(x, n)), (n, n_tok)


def test_quantize_ties_and_edges():
    # halves on an exact grid (away from zero), a negative maximum, tiny
    # scales (binary16 subnormal d) and large ones
    rows = []
    b = np.zeros(32, np.float32)
    b[:8] = [127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.49, 126.5]
    rows.append(b)
    rows.append(np.float32([-254, 3, 1, -5] + [0] * 28))
    rng = np.random.default_rng(3001)
    for s in (1e-6, 3e-5, 1e3, 4e6):
        rows.append((rng.standard_normal(32) * s).astype(np.float32))
    k = rng.integers(-127, 128, 32).astype(np.float32)
    k[5] = 127
    rows.append((k + 0.5 * np.sign(k)) * np.float32(2.0 ** -3))       # on-grid halves
    x = np.concatenate(rows).reshape(1, -1)
    assert np.array_equal(_gpu_blocks(x, x.size), _oracle_blocks(x, x.size))


SHAPES = {"q4_0": [(1, 32), (131, 576), (200, 1536), (97, 5120), (33, 17408)],
          "q8_0": [(1, 32), (45, 576), (130, 2048), (67, 4096)]}


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_q8act_within_bound(fmt):
    for k, (rows, cols) in enumerate(SHAPES[fmt]):
        rng = np.random.default_rng(3100 + k)
        t = synth.make_tensor(fmt, rows, cols, rng)
        x = rng.standard_normal((2, cols)).astype(np.float32)
        xd = G.torch.from_numpy(x).to(G.dev())
        y = G.qg().qgemv_q8act(fmt, G.upload(t), xd, rows, cols)
        G.torch.cuda.synchronize()
        yr, S = oracle.gemv_q8act(fmt, t.raw, x, rows, cols)
        G.check_bound(y.cpu().numpy(), yr, S, what=f"q8act {fmt} {rows}x{cols}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_q8act_exact_inputs_bit_exact(fmt):
    # power-of-two weight scales, activations k * 2^-4 with a code of 127 in
    # every block (so d_x = 2^-4 and the codes are k): every sum is exact
    rng = np.random.default_rng(3200)
    rows, cols = 150, 1024
    if fmt == "q4_0":
        d = (2.0 ** rng.integers(-6, -2, (rows, cols // 32))).astype(np.float16)
        raw = synth.pack_q4_0(d, rng.integers(0, 16, (rows, cols)))
    else:
        d = (2.0 ** rng.integers(-8, -4, (rows, cols // 32))).astype(np.float16)
        raw = synth.pack_q8_0(d, rng.integers(-127, 128, (rows, cols)).astype(np.int8))
    t = synth.QTensor("w", fmt, rows, cols, raw)
    kx = rng.integers(-127, 128, cols)
    kx[::32] = 127
    x = (kx * 2.0 ** -4).astype(np.float32)
    xd = G.torch.from_numpy(x).to(G.dev())
    y = G.qg().qgemv_q8act(fmt, G.upload(t), xd, rows, cols)
    G.torch.cuda.synchronize()
    yr, _ = oracle.gemv_q8act(fmt, t.raw, x, rows, cols)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), yr)


@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 288), (131, 576), (203, 5120), (33, 17408)])
def test_gemv_q8act_row_streaming_every_config(rows, cols):
    # Q4_0 weights at one token run on the row-streaming kernel, each lane
    # quantizing its own chunk of x: exact inputs (power-of-two weight scales,
    # activations on the Q8_0 grid) bit-identical to the oracle under the
    # built-in and every forced launch shape; random inputs within the bound
    # on it and on the lane-group kernel (qgemv_set_xs_override(-1))
    from tests.test_gpu_xs import _cfgs
    rng = np.random.default_rng(3250 + cols)
    d = (2.0 ** rng.integers(-6, -2, (rows, cols // 32))).astype(np.float16)
    t = synth.QTensor("w", "q4_0", rows, cols, synth.pack_q4_0(d, rng.integers(0, 16, (rows, cols))))
    pk = G.upload(t)
    kx = rng.integers(-127, 128, cols)
    kx[::32] = 127
    x = (kx * 2.0 ** -4).astype(np.float32)
    xd = G.torch.from_numpy(x).to(G.dev())
    yr, _ = oracle.gemv_q8act("q4_0", t.raw, x, rows, cols)
    cfgs = [None] + _cfgs(cols // 32, 1)[::3]
    try:
        for cfg in cfgs:
            if cfg is None:
                G.qg().set_xs_override(0)
            else:
                G.qg().set_xs_override(1, *cfg)
            y = G.qg().qgemv_q8act("q4_0", pk, xd, rows, cols)
            G.torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy().astype(np.float64), yr), f"{rows}x{cols} cfg {cfg}"
        tr = synth.make_tensor("q4_0", rows, cols, rng)
        pr = G.upload(tr)
        xr = rng.standard_normal(cols).astype(np.float32)
        yr2, S = oracle.gemv_q8act("q4_0", tr.raw, xr, rows, cols)
        for mode in (0, -1):
            G.qg().set_xs_override(mode)
            y = G.qg().qgemv_q8act("q4_0", pr, G.torch.from_numpy(xr).to(G.dev()), rows, cols)
            G.torch.cuda.synchronize()
            G.check_bound(y.cpu().numpy(), yr2, S, what=f"q8act {rows}x{cols} xs mode {mode}")
    finally:
        G.qg().set_xs_override(0)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_q8act_every_launch_shape(fmt):
    rows, cols = 203, 1536
    rng = np.random.default_rng(3300)
    t = synth.make_tensor(fmt, rows, cols, rng)
    pk = G.upload(t)
    x = rng.standard_normal(cols).astype(np.float32)
    xd = G.torch.from_numpy(x).to(G.dev())
    yr, S = oracle.gemv_q8act(fmt, t.raw, x, rows, cols)
    ref = None
    try:
        for lpr in (8, 16, 32, 64):
            for r in (1, 2):
                for waves, depth, max_wg in ((1, 2, 0), (4, 4, 3), (8, 2, 0)):
                    for cpl in (1, 2, 4):
                        G.qg().set_launch_override(lpr, r, waves, depth, max_wg, cpl)
                        y = G.qg().qgemv_q8act(fmt, pk, xd, rows, cols)
                        G.torch.cuda.synchronize()
                        G.check_bound(y.cpu().numpy(), yr, S, what=f"q8act {fmt} {lpr} {r} {waves} {depth} {cpl}")
    finally:
        G.qg().set_launch_override(0)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_q8act_deterministic_and_scale_invariant(fmt):
    # scaling x by 2 doubles every d_x exactly and leaves the codes: y doubles exactly
    rows, cols = 300, 2048
    rng = np.random.default_rng(3400)
    t = synth.make_tensor(fmt, rows, cols, rng)
    pk = G.upload(t)
    x = rng.standard_normal(cols).astype(np.float32)
    run = lambda v: G.qg().qgemv_q8act(fmt, pk, G.torch.from_numpy(v).to(G.dev()), rows, cols).cpu().numpy()
    y1, y2, y4 = run(x), run(x), run(x * np.float32(4))
    assert np.array_equal(y1, y2) and np.array_equal(y4, np.float32(4) * y1)


def _check_ffn_q8act(fmt, tens, x, d_model, ffn, what):
    pk = [G.upload(t) for t in tens]
    xd = G.torch.from_numpy(x).to(G.dev())
    out, h = G.qg().swiglu_ffn_q8act(fmt, pk[0], pk[1], pk[2], xd, d_model, ffn)
    G.torch.cuda.synchronize()
    out, h = out.cpu().numpy(), h.cpu().numpy()
    r = {}
    r["g"], r["Sg"] = oracle.gemv_q8act(fmt, tens[0].raw, x, ffn, d_model)
    r["u"], r["Su"] = oracle.gemv_q8act(fmt, tens[1].raw, x, ffn, d_model)
    r["h"] = G.silu64(r["g"]) * r["u"]
    assert np.all(np.abs(h - r["h"]) <= G.h_bound(r)), f"{what}: h outside its bound"
    yr, S = oracle.gemv_q8act(fmt, tens[2].raw, h, d_model, ffn)
    G.check_bound(out, yr, S, what=f"{what} down")


@pytest.mark.parametrize("fmt,n_tok", [("q4_0", 1), ("q8_0", 1), ("q4_0", 3)])
def test_swiglu_ffn_q8act(fmt, n_tok):
    d_model, ffn = 576, 1536
    rng = np.random.default_rng(3500 + n_tok)
    tens = [synth.make_tensor(fmt, ffn, d_model, rng), synth.make_tensor(fmt, ffn, d_model, rng),
            synth.make_tensor(fmt, d_model, ffn, rng)]
    x = rng.standard_normal((n_tok, d_model)).astype(np.float32)
    _check_ffn_q8act(fmt, tens, x, d_model, ffn, f"ffn q8act {fmt} n_tok={n_tok}")


@pytest.mark.parametrize("idx", range(8))
def test_fullsize_smollm2_layer_and_head_q8act(idx):
    # the SmolLM2-135M-shaped Q4_0 layer and its Q8_0 vocab head (the model the
    # mode was written for), every matrix at full size
    w = synth.CFG2
    t = synth.gen_tensor(w, idx)
    x = synth.gen_x(w, t.cols, 1, which=idx)
    xd = G.torch.from_numpy(x).to(G.dev())
    y = G.qg().qgemv_q8act(t.fmt, G.upload(t), xd, t.rows, t.cols)
    G.torch.cuda.synchronize()
    yr, S = oracle.gemv_q8act(t.fmt, t.raw, x, t.rows, t.cols)
    G.check_bound(y.cpu().numpy(), yr, S, what=f"cfg2 {t.name} q8act")


def test_fullsize_27b_ffn_q8act():
    w = synth.CFG5
    tens = synth.gen_workload(w)
    x = synth.gen_x(w, w.d_model, 1)
    _check_ffn_q8act("q4_0", tens, x, w.d_model, w.ffn, "27B-class FFN q8act")


# ---- several tokens: one launch per product on the matrix cores ----------
#
# The batched path quantizes each token's x blocks inside the kernel with the
# same rule and multiplies the codes on the matrix cores (binary16 integer
# operands, exact fp32 block sums), then scales each block sum by d_w * d_x:
# the same fp32 bound as one token.

def _oracle_q8act_rows(fmt, raw, x, rows, cols, threads=16):
    """oracle.gemv_q8act over row ranges on a thread pool (the raw blocks of
    Q4_0 and Q8_0 are whole rows in order, so a range is a slice; each row's
    sum is the same as in one call)."""
    from concurrent.futures import ThreadPoolExecutor
    rb = (cols // 32) * (18 if fmt == "q4_0" else 34)
    raw = np.ascontiguousarray(raw).reshape(rows, rb)
    threads = max(1, min(threads, rows // 64 or 1))
    cuts = np.linspace(0, rows, threads + 1).astype(int)
    with ThreadPoolExecutor(threads) as pool:
        parts = list(pool.map(lambda ab: oracle.gemv_q8act(fmt, raw[ab[0]:ab[1]].reshape(-1), x, int(ab[1] - ab[0]),
                                                           cols), zip(cuts[:-1], cuts[1:])))
    return np.concatenate([p[0] for p in parts], axis=-1), np.concatenate([p[1] for p in parts], axis=-1)


BATCH_SHAPES = {"q4_0": [(1, 32), (45, 576), (203, 1536), (64, 4096), (130, 160)],
                "q8_0": [(1, 32), (45, 576), (131, 2048), (67, 1056)]}


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n_tok", [2, 3, 16, 17, 40, 70])
def test_gemv_q8act_batched_within_bound(fmt, n_tok):
    for k, (rows, cols) in enumerate(BATCH_SHAPES[fmt]):
        rng = np.random.default_rng(3600 + 10 * n_tok + k)
        t = synth.make_tensor(fmt, rows, cols, rng)
        x = rng.standard_normal((n_tok, cols)).astype(np.float32)
        x[n_tok // 2, :32] = 0.0                                        # a zero block
        y = G.qg().qgemv_q8act(fmt, G.upload(t), G.torch.from_numpy(x).to(G.dev()), rows, cols)
        G.torch.cuda.synchronize()
        yr, S = oracle.gemv_q8act(fmt, t.raw, x, rows, cols)
        G.check_bound(y.cpu().numpy(), yr, S, what=f"q8act batched {fmt} {rows}x{cols} n_tok={n_tok}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_q8act_batched_every_tile(fmt):
    # every built tile, K unsplit, split in 3 and 7, and as many ranges as
    # super-steps (33 asked, 9 taken: 1056 columns are 33 blocks)
    rows, cols, n_tok = 203, 1056, 37
    rng = np.random.default_rng(3700)
    t = synth.make_tensor(fmt, rows, cols, rng)
    pk = G.upload(t)
    x = rng.standard_normal((n_tok, cols)).astype(np.float32)
    xd = G.torch.from_numpy(x).to(G.dev())
    yr, S = oracle.gemv_q8act(fmt, t.raw, x, rows, cols)
    try:
        for mtr, ntw, ks in ((1, 1, 0), (1, 2, 0), (1, 4, 0), (2, 1, 0), (2, 2, 0), (2, 4, 0), (1, 1, 1), (1, 1, 3),
                             (2, 4, 7), (1, 2, 33)):
            G.qg().set_prefill_override(mtr, ntw, 4, 1, ks)
            y = G.qg().qgemv_q8act(fmt, pk, xd, rows, cols)
            G.torch.cuda.synchronize()
            G.check_bound(y.cpu().numpy(), yr, S, what=f"q8act batched {fmt} tile {mtr} {ntw} ksplit {ks}")
    finally:
        G.qg().set_prefill_override(0)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_q8act_batched_exact_inputs_bit_exact(fmt):
    # power-of-two weight scales, activations k * 2^-e with a code of 127 in
    # every block: each block sum is an exact integer times a power of two and
    # every partial sum is exact, so y equals the oracle's bit for bit
    rng = np.random.default_rng(3800)
    rows, cols, n_tok = 150, 1024, 21
    if fmt == "q4_0":
        d = (2.0 ** rng.integers(-6, -2, (rows, cols // 32))).astype(np.float16)
        raw = synth.pack_q4_0(d, rng.integers(0, 16, (rows, cols)))
    else:
        d = (2.0 ** rng.integers(-8, -4, (rows, cols // 32))).astype(np.float16)
        raw = synth.pack_q8_0(d, rng.integers(-127, 128, (rows, cols)).astype(np.int8))
    t = synth.QTensor("w", fmt, rows, cols, raw)
    kx = rng.integers(-127, 128, (n_tok, cols))
    kx[:, ::32] = 127
    x = (kx * 2.0 ** -rng.integers(3, 6, (n_tok, 1))).astype(np.float32)
    y = G.qg().qgemv_q8act(fmt, G.upload(t), G.torch.from_numpy(x).to(G.dev()), rows, cols)
    G.torch.cuda.synchronize()
    yr, _ = oracle.gemv_q8act(fmt, t.raw, x, rows, cols)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), yr)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_q8act_batched_matches_token_loop_scaled(fmt):
    # the batched launch against the per-token GEMV loop (both within the
    # bound of the oracle), and exact doubling when x doubles
    rows, cols, n_tok = 300, 2048, 24
    rng = np.random.default_rng(3900)
    t = synth.make_tensor(fmt, rows, cols, rng)
    pk = G.upload(t)
    x = rng.standard_normal((n_tok, cols)).astype(np.float32)
    run = lambda v: G.qg().qgemv_q8act(fmt, pk, G.torch.from_numpy(v).to(G.dev()), rows, cols).cpu().numpy()
    yb, yb2, y4 = run(x), run(x), run(x * np.float32(4))
    assert np.array_equal(yb, yb2) and np.array_equal(y4, np.float32(4) * yb)
    try:
        G.qg().set_prefill_override(-1)
        yl = run(x)
    finally:
        G.qg().set_prefill_override(0)
    yr, S = oracle.gemv_q8act(fmt, t.raw, x, rows, cols)
    G.check_bound(yb, yr, S, what="batched")
    G.check_bound(yl, yr, S, what="token loop")


def test_gemv_q8act_batched_workspace_sizes():
    # the workspace's size decides the K split only: the least that holds the
    # quantized activations, and more, give results within the bound; less
    # is refused
    fmt, rows, cols, n_tok = "q4_0", 130, 2048, 20
    rng = np.random.default_rng(4100)
    t = synth.make_tensor(fmt, rows, cols, rng)
    pk = G.upload(t)
    x = rng.standard_normal((n_tok, cols)).astype(np.float32)
    xd = G.torch.from_numpy(x).to(G.dev())
    yr, S = oracle.gemv_q8act(fmt, t.raw, x, rows, cols)
    xb = n_tok * (cols // 32) * 64 + n_tok * (cols // 32) * 4          # both multiples of 256 here
    full = G.qg().q8act_workspace_bytes(fmt, rows, cols, n_tok)
    assert full > xb
    for nb in (xb, xb + 3 * 4 * rows * n_tok, full, full + 4096):
        ws = G.torch.empty(nb, dtype=G.torch.uint8, device=G.dev())
        y = G.qg().qgemv_q8act(fmt, pk, xd, rows, cols, workspace=ws)
        G.torch.cuda.synchronize()
        G.check_bound(y.cpu().numpy(), yr, S, what=f"workspace {nb}")
    with pytest.raises(G.qg().QGemvError):
        G.qg().qgemv_q8act(fmt, pk, xd, rows, cols, workspace=G.torch.empty(xb - 256, dtype=G.torch.uint8,
                                                                             device=G.dev()))


def test_swiglu_ffn_q8act_scratch_sizes():
    # h_scratch of n_tok * ffn floats: the per-token loop; the full size: the
    # batched launches; both within the bounds, stage by stage
    fmt, d_model, ffn, n_tok = "q8_0", 576, 1536, 12
    rng = np.random.default_rng(4200)
    tens = [synth.make_tensor(fmt, ffn, d_model, rng), synth.make_tensor(fmt, ffn, d_model, rng),
            synth.make_tensor(fmt, d_model, ffn, rng)]
    pk = [G.upload(t) for t in tens]
    x = rng.standard_normal((n_tok, d_model)).astype(np.float32)
    xd = G.torch.from_numpy(x).to(G.dev())
    for elems in (n_tok * ffn, G.qg().swiglu_ffn_q8act_scratch_elems(fmt, d_model, ffn, n_tok)):
        h_s = G.torch.empty(elems, dtype=G.torch.float32, device=G.dev())
        out, h = G.qg().swiglu_ffn_q8act(fmt, pk[0], pk[1], pk[2], xd, d_model, ffn, h_scratch=h_s)
        G.torch.cuda.synchronize()
        out, h = out.cpu().numpy(), h.cpu().numpy()
        r = {}
        r["g"], r["Sg"] = oracle.gemv_q8act(fmt, tens[0].raw, x, ffn, d_model)
        r["u"], r["Su"] = oracle.gemv_q8act(fmt, tens[1].raw, x, ffn, d_model)
        r["h"] = G.silu64(r["g"]) * r["u"]
        assert np.all(np.abs(h - r["h"]) <= G.h_bound(r)), f"scratch {elems}: h outside its bound"
        yr, S = oracle.gemv_q8act(fmt, tens[2].raw, h, d_model, ffn)
        G.check_bound(out, yr, S, what=f"scratch {elems} down")


@pytest.mark.parametrize("fmt,n_tok", [("q4_0", 8), ("q8_0", 17), ("q4_0", 40)])
def test_swiglu_ffn_q8act_batched(fmt, n_tok):
    d_model, ffn = 576, 1536
    rng = np.random.default_rng(4000 + n_tok)
    tens = [synth.make_tensor(fmt, ffn, d_model, rng), synth.make_tensor(fmt, ffn, d_model, rng),
            synth.make_tensor(fmt, d_model, ffn, rng)]
    x = rng.standard_normal((n_tok, d_model)).astype(np.float32)
    _check_ffn_q8act(fmt, tens, x, d_model, ffn, f"ffn q8act {fmt} n_tok={n_tok}")


@pytest.mark.parametrize("n_tok", [8, 128])
def test_fullsize_27b_ffn_q8act_batched_every_row(n_tok):
    w = synth.CFG5
    tens = synth.gen_workload(w)
    x = synth.gen_x(w, w.d_model, n_tok)
    pk = [G.upload(t) for t in tens]
    out, h = G.qg().swiglu_ffn_q8act("q4_0", pk[0], pk[1], pk[2], G.torch.from_numpy(x).to(G.dev()), w.d_model,
                                     w.ffn)
    G.torch.cuda.synchronize()
    out, h = out.cpu().numpy(), h.cpu().numpy()
    r = {}
    r["g"], r["Sg"] = _oracle_q8act_rows("q4_0", tens[0].raw, x, w.ffn, w.d_model)
    r["u"], r["Su"] = _oracle_q8act_rows("q4_0", tens[1].raw, x, w.ffn, w.d_model)
    r["h"] = G.silu64(r["g"]) * r["u"]
    assert np.all(np.abs(h - r["h"]) <= G.h_bound(r)), f"27B q8act n_tok={n_tok}: h outside its bound"
    yr, S = _oracle_q8act_rows("q4_0", tens[2].raw, h, w.d_model, w.ffn)
    G.check_bound(out, yr, S, what=f"27B q8act n_tok={n_tok} down")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n_tok", [5, 20])
def test_gemv_q8act_batched_edge_scales_within_bound(fmt, n_tok):
    # every row's weight scales in one binary16 binade (subnormal to the top,
    # either sign, some zeros), Q8_0 codes over -128..127 (one row all -128)
    from tests.test_gpu_scale_edges import make, row_binade_f16
    rows, cols = 131, 2048
    rng = np.random.default_rng(4500 + 10 * FMTS.index(fmt) + n_tok)
    t = make(fmt, rows, cols, rng, row_binade_f16)
    x = rng.standard_normal((n_tok, cols)).astype(np.float32)
    y = G.qg().qgemv_q8act(fmt, G.upload(t), G.torch.from_numpy(x).to(G.dev()), rows, cols)
    G.torch.cuda.synchronize()
    yr, S = oracle.gemv_q8act(fmt, t.raw, x, rows, cols)
    G.check_bound(y.cpu().numpy(), yr, S, what=f"q8act batched {fmt} edge scales n_tok={n_tok}")


def test_gemv_q8act_batched_extreme_codes_bit_exact():
    # Q8_0 weight codes at the ends of the range (-128, -127, 127, 0) and
    # activation codes of +-127, one power-of-two scale for all weights and
    # one for all activations: y = 2^-11 * sum q k, whose every partial sum
    # is an integer of at most 1024 * 128 * 127 < 2^24 units, exact in fp32,
    # so y equals the oracle bit for bit; the decode of -128 (the byte 0x80)
    # included
    rng = np.random.default_rng(4600)
    rows, cols, n_tok = 77, 1024, 18
    d = np.full((rows, cols // 32), 2.0 ** -6, np.float16)
    q = rng.choice(np.array([-128, -127, 127, 0], np.int8), (rows, cols))
    q[5] = -128                                                          # the extreme row sums
    t = synth.QTensor("w", "q8_0", rows, cols, synth.pack_q8_0(d, q))
    kx = rng.choice(np.array([-127, 127]), (n_tok, cols))
    kx[3] = -127
    x = (kx * 2.0 ** -5).astype(np.float32)
    y = G.qg().qgemv_q8act("q8_0", G.upload(t), G.torch.from_numpy(x).to(G.dev()), rows, cols)
    G.torch.cuda.synchronize()
    yr, _ = oracle.gemv_q8act("q8_0", t.raw, x, rows, cols)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), yr)
