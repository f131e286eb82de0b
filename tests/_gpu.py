"""Shared helpers for the GPU parity tests: upload raw blocks, run the C ABI
through the binding, compare with the oracle under the stated bounds."""
import numpy as np
import torch

import oracle

REL = 2e-5      # fp32 GEMV bound: |dy| <= REL * sum|w x| + ABS
ABS = 1e-7
SILU_REL = 1e-6  # budget for the device exp and divide in h = silu(g) * u


def dev():
    return torch.device("cuda:0")


def qg():
    import dequant_matrix_vector_amd as m
    return m


def upload(t):
    """Packed device buffer of a synth.QTensor."""
    d = dev()
    raw = torch.from_numpy(np.ascontiguousarray(t.raw)).to(d)
    rs = None if t.row_scale is None else torch.from_numpy(t.row_scale).to(d)
    return qg().repack(t.fmt, raw, t.rows, t.cols, row_scale=rs)


def gemv_gpu(t, packed, x):
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())
    y = qg().qgemv(t.fmt, packed, xd, t.rows, t.cols)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check_bound(y_gpu, y_ref, S, rel=REL, what=""):
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ref)
    bound = rel * S + ABS
    bad = ~(err <= bound)
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside the bound; first flat index {i}: "
                             f"gpu {y_gpu.reshape(-1)[i]!r} ref {y_ref.reshape(-1)[i]!r} "
                             f"bound {bound.reshape(-1)[i]!r}")
    return float((err / bound).max()) if err.size else 0.0


def silu64(g):
    return g / (1.0 + np.exp(-g))


def h_bound(r):
    """Per-element bound on h = silu(g) u from the GEMV bounds of g and u."""
    g, u = r["g"], r["u"]
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    Bg = REL * r["Sg"] + ABS
    Bu = REL * r["Su"] + ABS
    return np.abs(dsilu * u) * Bg + np.abs(silu64(g)) * Bu + SILU_REL * np.abs(r["h"]) + 1e-30
