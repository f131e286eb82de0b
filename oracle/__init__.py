"""CPU oracle for the block-quantized GEMV and the SwiGLU FFN.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
bench.py's cpu_baseline leg, never by the product package.  It wraps the plain
scalar C in oracle.c (binary64 accumulation, sequential column order) through
ctypes and shares no code with the HIP library.

Formats (constants match the C side): Q4_0=0, Q8_0=1, Q4_K=2, I8ROW=3, Q6_K=4.
`raw` is the tensor's raw block bytes ([rows][cols/B] blocks, row-major) as a
uint8 numpy array; for I8ROW it is the int8 code matrix and `row_scale` holds the
fp32 per-row scales.
"""
import ctypes
import os

import numpy as np

from . import build as _build

Q4_0, Q8_0, Q4_K, I8ROW, Q6_K = 0, 1, 2, 3, 4
FORMATS = {"q4_0": Q4_0, "q8_0": Q8_0, "q4_k": Q4_K, "i8row": I8ROW, "q6_k": Q6_K}

_lib = None


def use_library(path=None):
    """Point the wrapper at another build of oracle.c (None: the default one).
    The mutation tests use this to run the pins against planted mistakes."""
    global _lib, _path
    _lib = None
    _path = path


# ORACLE_LIB lets the mutation tests run the whole pin suite in a child
# process against a deliberately broken build.
_path = os.environ.get("ORACLE_LIB") or None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _path is None:
        src = os.path.join(os.path.dirname(__file__), "oracle.c")
        if (not os.path.exists(_build.LIB)) or os.path.getmtime(_build.LIB) < os.path.getmtime(src):
            _build.build()
    lib = ctypes.CDLL(_path or _build.LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_q4k_scale_min.argtypes = [ctypes.c_int, P, P, P]
    lib.oracle_q4k_scale_min.restype = None
    lib.oracle_dequant.argtypes = [ctypes.c_int, P, P, I64, I64, P]
    lib.oracle_dequant.restype = ctypes.c_int
    lib.oracle_gemv.argtypes = [ctypes.c_int, P, P, P, I64, I64, I64, I64, I64, P, P]
    lib.oracle_gemv.restype = ctypes.c_int
    lib.oracle_gemv_f64x.argtypes = [ctypes.c_int, P, P, P, I64, I64, I64, P, P]
    lib.oracle_gemv_f64x.restype = ctypes.c_int
    lib.oracle_rmsnorm.argtypes = [P, P, I64, I64, ctypes.c_double, P, P]
    lib.oracle_rmsnorm.restype = ctypes.c_int
    lib.oracle_ffn_block.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, ctypes.c_double, P, I64, I64, I64,
                                     P, P, P, P, P, P, P, P, P]
    lib.oracle_ffn_block.restype = ctypes.c_int
    lib.oracle_argmax.argtypes = [P, I64]
    lib.oracle_argmax.restype = I64
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_quantize_q8_0.argtypes = [P, I64, I64, P, P]
    lib.oracle_quantize_q8_0.restype = ctypes.c_int
    lib.oracle_gemv_q8act.argtypes = [ctypes.c_int, P, P, I64, I64, I64, P, P]
    lib.oracle_gemv_q8act.restype = ctypes.c_int
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_swiglu.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, I64, I64, I64,
                                  P, P, P, P, P, P, P]
    lib.oracle_swiglu.restype = ctypes.c_int
    _lib = lib
    return lib


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _raw(raw):
    a = np.ascontiguousarray(raw)
    return a


def _scale(row_scale):
    return None if row_scale is None else np.ascontiguousarray(row_scale, dtype=np.float32)


def _check(st, what):
    if st != 0:
        raise ValueError(f"oracle {what} failed with status {st}")


def f16_to_f64(h: int) -> float:
    return _load().oracle_f16_to_f64(int(h) & 0xFFFF)


def q4k_scale_min(j: int, scales12) -> tuple:
    b = np.ascontiguousarray(np.asarray(scales12, dtype=np.uint8))
    assert b.size == 12
    sc = ctypes.c_int()
    m = ctypes.c_int()
    _load().oracle_q4k_scale_min(int(j), _ptr(b), ctypes.byref(sc), ctypes.byref(m))
    return sc.value, m.value


def silu(g: float) -> float:
    return _load().oracle_silu(float(g))


def dequant(fmt, raw, rows, cols, row_scale=None) -> np.ndarray:
    """fp32 [rows][cols]: every weight rounded once (RNE) from its exact value."""
    raw = _raw(raw)
    rs = _scale(row_scale)
    out = np.empty((rows, cols), dtype=np.float32)
    _check(_load().oracle_dequant(_fmt(fmt), _ptr(raw), _ptr(rs), rows, cols, _ptr(out)), "dequant")
    return out


def gemv(fmt, raw, x, rows, cols, row_scale=None, row_begin=0, row_end=None):
    """(y, S), both float64 [n_tok][nrows]; x is float32 [n_tok][cols] (or [cols])."""
    raw = _raw(raw)
    rs = _scale(row_scale)
    x = np.ascontiguousarray(x, dtype=np.float32)
    squeeze = x.ndim == 1
    x2 = x.reshape(-1, cols)
    n_tok = x2.shape[0]
    row_end = rows if row_end is None else row_end
    nr = row_end - row_begin
    y = np.empty((n_tok, nr), dtype=np.float64)
    S = np.empty((n_tok, nr), dtype=np.float64)
    _check(_load().oracle_gemv(_fmt(fmt), _ptr(raw), _ptr(rs), _ptr(x2), rows, cols, n_tok,
                               row_begin, row_end, _ptr(y), _ptr(S)), "gemv")
    if squeeze:
        return y[0], S[0]
    return y, S


def gemv_f64x(fmt, raw, x64, rows, cols, row_scale=None):
    """Same product with a float64 right-hand side [n_tok][cols]."""
    raw = _raw(raw)
    rs = _scale(row_scale)
    x = np.ascontiguousarray(x64, dtype=np.float64).reshape(-1, cols)
    n_tok = x.shape[0]
    y = np.empty((n_tok, rows), dtype=np.float64)
    S = np.empty((n_tok, rows), dtype=np.float64)
    _check(_load().oracle_gemv_f64x(_fmt(fmt), _ptr(raw), _ptr(rs), _ptr(x), rows, cols, n_tok,
                                    _ptr(y), _ptr(S)), "gemv_f64x")
    return y, S


def swiglu(fmt, wg, wu, wd, x, d_model, ffn, sg=None, su=None, sd=None):
    """Dict of float64 arrays g, u, h, out, Sg, Su, Sd (token-major)."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, d_model)
    n_tok = x.shape[0]
    r = {k: np.empty((n_tok, ffn), dtype=np.float64) for k in ("g", "u", "h", "Sg", "Su")}
    r["out"] = np.empty((n_tok, d_model), dtype=np.float64)
    r["Sd"] = np.empty((n_tok, d_model), dtype=np.float64)
    wg, wu, wd = _raw(wg), _raw(wu), _raw(wd)
    sg, su, sd = _scale(sg), _scale(su), _scale(sd)
    _check(_load().oracle_swiglu(_fmt(fmt), _ptr(wg), _ptr(sg), _ptr(wu), _ptr(su), _ptr(wd),
                                 _ptr(sd), _ptr(x), d_model, ffn, n_tok,
                                 _ptr(r["g"]), _ptr(r["u"]), _ptr(r["h"]), _ptr(r["out"]),
                                 _ptr(r["Sg"]), _ptr(r["Su"]), _ptr(r["Sd"])), "swiglu")
    return r


def rmsnorm(x, gamma, eps):
    """(xn, scale): float64 [n_tok][n] and [n_tok] for float32 x [n_tok][n] (or [n])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    squeeze = x.ndim == 1
    n = x.shape[-1]
    x2 = x.reshape(-1, n)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    assert gamma.shape == (n,)
    out = np.empty(x2.shape, dtype=np.float64)
    scale = np.empty(x2.shape[0], dtype=np.float64)
    _check(_load().oracle_rmsnorm(_ptr(x2), _ptr(gamma), n, x2.shape[0], float(eps), _ptr(out), _ptr(scale)),
           "rmsnorm")
    return (out[0], scale[0]) if squeeze else (out, scale)


def ffn_block(fmt, wg, wu, wd, gamma, eps, x, d_model, ffn, sg=None, su=None, sd=None):
    """Dict of float64 arrays xn, g, u, h, d, out, Sg, Su, Sd: out = x + Wd(silu(Wg xn)(Wu xn)),
    xn = rmsnorm(x) * gamma."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, d_model)
    n_tok = x.shape[0]
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    r = {k: np.empty((n_tok, ffn), dtype=np.float64) for k in ("g", "u", "h", "Sg", "Su")}
    for k in ("xn", "d", "out", "Sd"):
        r[k] = np.empty((n_tok, d_model), dtype=np.float64)
    wg, wu, wd = _raw(wg), _raw(wu), _raw(wd)
    sg, su, sd = _scale(sg), _scale(su), _scale(sd)
    _check(_load().oracle_ffn_block(_fmt(fmt), _ptr(wg), _ptr(sg), _ptr(wu), _ptr(su), _ptr(wd), _ptr(sd),
                                    _ptr(gamma), float(eps), _ptr(x), d_model, ffn, n_tok,
                                    _ptr(r["xn"]), _ptr(r["g"]), _ptr(r["u"]), _ptr(r["h"]), _ptr(r["d"]),
                                    _ptr(r["out"]), _ptr(r["Sg"]), _ptr(r["Su"]), _ptr(r["Sd"])), "ffn_block")
    return r


def argmax(v) -> int:
    """First index of the largest value of a float32 vector (greedy sampling)."""
    v = np.ascontiguousarray(v, dtype=np.float32).reshape(-1)
    r = _load().oracle_argmax(_ptr(v), v.size)
    if r < 0:
        raise ValueError(f"oracle argmax: status {r}")
    return int(r)


def f32_to_f16(f) -> int:
    """binary16 bits of a binary32 value, round to nearest even."""
    return int(_load().oracle_f32_to_f16(float(np.float32(f))))


def quantize_q8_0(x):
    """Q8_0 blocks of activation rows: (d_bits uint16 [n_tok][n/32], q int8 [n_tok][n])
    for float32 x [n_tok][n] (or [n])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    squeeze = x.ndim == 1
    n = x.shape[-1]
    x2 = x.reshape(-1, n)
    d = np.empty((x2.shape[0], n // 32), dtype=np.uint16)
    q = np.empty(x2.shape, dtype=np.int8)
    _check(_load().oracle_quantize_q8_0(_ptr(x2), n, x2.shape[0], _ptr(d), _ptr(q)), "quantize_q8_0")
    return (d[0], q[0]) if squeeze else (d, q)


def gemv_q8act(fmt, raw, x, rows, cols):
    """(y, S) float64 [n_tok][rows] of W times the Q8_0 representation of x."""
    raw = _raw(raw)
    x = np.ascontiguousarray(x, dtype=np.float32)
    squeeze = x.ndim == 1
    x2 = x.reshape(-1, cols)
    n_tok = x2.shape[0]
    y = np.empty((n_tok, rows), dtype=np.float64)
    S = np.empty((n_tok, rows), dtype=np.float64)
    _check(_load().oracle_gemv_q8act(_fmt(fmt), _ptr(raw), _ptr(x2), rows, cols, n_tok, _ptr(y), _ptr(S)),
           "gemv_q8act")
    return (y[0], S[0]) if squeeze else (y, S)
