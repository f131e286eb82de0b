"""Shared helpers for the GPU parity tests: upload raw blocks, run the C ABI
through the binding, compare with the oracle under the stated bounds."""
import numpy as np
import torch

import oracle

REL = 2e-5      # fp32 GEMV bound: |dy| <= REL * sum|w x| + ABS
ABS = 1e-7
SILU_REL = 1e-6  # budget for the device exp and divide in h = silu(g) * u
# matrix-core path (Q4_0 and Q4_K, n_tok > 1): weights and x rounded to bf16 (nearest
# even) before fp32 accumulation, each term off by at most about 2 * 2^-9
PF_REL = 8e-3


def rel_for(fmt, n_tok):
    """The bound's relative factor for a product of this format and batch."""
    return PF_REL if (fmt in ("q4_0", "q4_k", "q6_k", "q8_0", "i8row") and n_tok > 1) else REL


def bf16_rne(a):
    """float32 values rounded to bfloat16, nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


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


def oracle_gemv_rows(fmt, raw, x, rows, cols, row_scale=None, threads=16):
    """oracle.gemv over every row, the rows split into ranges run on a thread
    pool (ctypes releases the GIL in the C oracle; each row is summed in the
    same order as in one call, so the result is identical)."""
    from concurrent.futures import ThreadPoolExecutor
    threads = max(1, min(threads, rows // 64 or 1))
    cuts = np.linspace(0, rows, threads + 1).astype(int)
    with ThreadPoolExecutor(threads) as pool:
        parts = list(pool.map(lambda ab: oracle.gemv(fmt, raw, x, rows, cols, row_scale=row_scale,
                                                     row_begin=int(ab[0]), row_end=int(ab[1])),
                              zip(cuts[:-1], cuts[1:])))
    y = np.concatenate([p[0] for p in parts], axis=-1)
    S = np.concatenate([p[1] for p in parts], axis=-1)
    return y, S


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


def h_bound(r, rel=REL):
    """Per-element bound on h = silu(g) u from the product bounds of g and u."""
    g, u = r["g"], r["u"]
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    Bg = rel * r["Sg"] + ABS
    Bu = rel * r["Su"] + ABS
    return np.abs(dsilu * u) * Bg + np.abs(silu64(g)) * Bu + SILU_REL * np.abs(r["h"]) + 1e-30


def check_ffn(fmt, tens, x, d_model, ffn, what):
    rel = rel_for(fmt, x.shape[0])
    g, u, d = tens
    pk = [upload(t) for t in tens]
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(dev())
    out, h = qg().swiglu_ffn(fmt, pk[0], pk[1], pk[2], xd, d_model, ffn)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    h = h.cpu().numpy()
    r = oracle.swiglu(fmt, g.raw, u.raw, d.raw, x, d_model, ffn, g.row_scale, u.row_scale, d.row_scale)
    # stage 1: h against silu(g) u of the oracle
    hb = h_bound(r, rel)
    assert np.all(np.abs(h - r["h"]) <= hb), f"{what}: h outside its bound"
    # stage 2: out against the oracle's down projection of the device's own h
    yr, S = oracle.gemv(fmt, d.raw, h, d_model, ffn, row_scale=d.row_scale)
    check_bound(out, yr, S, rel=rel, what=f"{what} down")
    return out, h, r, hb
