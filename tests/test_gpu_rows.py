"""GPU parity of the row-packed one-token kernel (Q8_0 rows of at most 64
blocks: one lane per block position, rows laid across the lanes) through the
C ABI, against the oracle: |y_gpu - y_ref| <= 2e-5 * sum_j |w_ij x_j| + 1e-7.

Its launch shape is forced through qgemv_set_xs_override (ring depth, row-steps
per workgroup, workgroups per CU) so that every tail of the ring (1 to depth
row-steps after the last full batch), idle lanes (threads that hold no whole
row) and a partial last row-step are run; the lane-group kernels
(override -1) give a second product within the same bound.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu

# (rows, cols): 18 blocks (no idle lane at 9 waves), 1, 3, 31, 33, 64 blocks
SHAPES = [(49, 576), (300, 32), (257, 96), (77, 992), (130, 1056), (90, 2048)]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_rows_kernel_every_shape(rows, cols):
    rng = np.random.default_rng(4300 + cols)
    t = synth.make_tensor("q8_0", rows, cols, rng)
    pk = G.upload(t)
    x = rng.standard_normal(cols).astype(np.float32)
    xd = G.torch.from_numpy(x).to(G.dev())
    yr, S = oracle.gemv("q8_0", t.raw, x, rows, cols)
    try:
        for depth, nrs, wpc in ((0, 0, -1), (2, 1, -1), (2, 3, -1), (4, 5, -1), (4, 4, -1), (8, 7, -1), (8, 9, -1),
                                (4, 0, 3), (2, 0, 1)):
            if depth == 0:
                G.qg().set_xs_override(0)
            else:
                G.qg().set_xs_override(1, 0, 0, depth, nrs, -1, wpc)
            y = G.qg().qgemv("q8_0", pk, xd, rows, cols)
            G.torch.cuda.synchronize()
            G.check_bound(y.cpu().numpy(), yr, S, what=f"rows {rows}x{cols} depth {depth} nrs {nrs} wpc {wpc}")
        G.qg().set_xs_override(-1)
        y = G.qg().qgemv("q8_0", pk, xd, rows, cols)
        G.torch.cuda.synchronize()
        G.check_bound(y.cpu().numpy(), yr, S, what=f"lane groups {rows}x{cols}")
    finally:
        G.qg().set_xs_override(0)


def test_rows_kernel_head_argmax_every_depth():
    # the fused greedy sampling on this kernel: ties at the largest value
    # resolved to the first index, at each ring depth
    rows, cols = 3000, 576
    rng = np.random.default_rng(4400)
    nb = cols // 32
    d = rng.uniform(0.005, 0.05, (rows, nb)).astype(np.float16)
    q = rng.integers(-60, 61, (rows, cols)).astype(np.int8)
    q[[17, 1800, 2999]] = 127                 # three equal rows with the largest products
    d[[17, 1800, 2999]] = np.float16(0.06)
    raw = synth.pack_q8_0(d, q)
    t = synth.QTensor("head", "q8_0", rows, cols, raw)
    pk = G.upload(t)
    x = np.abs(rng.standard_normal(cols)).astype(np.float32)
    xd = G.torch.from_numpy(x).to(G.dev())
    try:
        for depth in (2, 4, 8):
            G.qg().set_xs_override(1, 0, 0, depth, 0, -1, -1)
            tok, logits = G.qg().qgemv_head_argmax("q8_0", pk, xd, rows, cols, fused=True)
            G.torch.cuda.synchronize()
            assert int(tok.cpu()[0]) == 17, depth
            lg = logits.cpu().numpy().reshape(-1)
            assert int(tok.cpu()[0]) == oracle.argmax(lg)
    finally:
        G.qg().set_xs_override(0)
