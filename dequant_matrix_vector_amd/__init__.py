"""Python binding of libqgemv.so (the C ABI declared in include/qgemv.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's gfx950
kernels.  The entry points keep the C names (qgemv_q4_0, swiglu_ffn, qdequant,
qgemv_repack_q4_0, ...) and raise QGemvError on a nonzero status.  There is no
CPU fallback: if the library is missing, importing this module fails.
"""
import ctypes
import os

import torch

__all__ = [
    "FORMATS", "QGemvError", "lib", "packed_bytes", "max_cols", "repack",
    "qgemv", "qgemv_q4_0", "qgemv_q8_0", "qgemv_q4_k", "qgemv_i8row", "qgemv_q6_k",
    "swiglu_gate_up", "swiglu_ffn", "swiglu_ffn_noalloc", "qdequant", "layout_version", "set_launch_override",
    "set_prefill_override", "set_xs_override", "set_ffn_khalf", "prefill_plan", "swiglu_ffn_scratch_elems", "swiglu_ffn_block", "swiglu_ffn_block_scratch_elems",
    "qgemv_argmax", "qgemv_head_argmax", "head_argmax_workspace_bytes", "qgemv_q8act", "swiglu_ffn_q8act", "q8act_workspace_bytes",
    "swiglu_ffn_q8act_scratch_elems", "qquantize_q8_0",
    "qgemv_repack_q4_0", "qgemv_repack_q8_0", "qgemv_repack_q4_k", "qgemv_repack_i8row", "qgemv_repack_q6_k",
]

FORMATS = {"q4_0": 0, "q8_0": 1, "q4_k": 2, "i8row": 3, "q6_k": 4}
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")

lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int

lib.qgemv_layout_version.restype = _I
lib.qgemv_status_string.argtypes = [_I]
lib.qgemv_status_string.restype = ctypes.c_char_p
lib.qgemv_max_cols.restype = _I64
lib.qgemv_packed_bytes.argtypes = [_I, _I64, _I64]
lib.qgemv_packed_bytes.restype = _I64
for _n in ("qgemv_repack_q4_0", "qgemv_repack_q8_0", "qgemv_repack_q4_k", "qgemv_repack_q6_k"):
    getattr(lib, _n).argtypes = [_P, _P, _I64, _I64, _P]
    getattr(lib, _n).restype = _I
lib.qgemv_repack_i8row.argtypes = [_P, _P, _P, _I64, _I64, _P]
lib.qgemv_repack_i8row.restype = _I
for _n in ("qgemv_q4_0", "qgemv_q8_0", "qgemv_q4_k", "qgemv_i8row", "qgemv_q6_k"):
    getattr(lib, _n).argtypes = [_P, _P, _P, _I64, _I64, _I64, _P]
    getattr(lib, _n).restype = _I
lib.qgemv.argtypes = [_I, _P, _P, _P, _I64, _I64, _I64, _P]
lib.qgemv_prefill_plan.argtypes = [_I, _I, _I64, _I64, _I64, _I64, _I, _P]
lib.qgemv.restype = _I
lib.swiglu_gate_up.argtypes = [_I, _P, _P, _P, _P, _I64, _I64, _I64, _P]
lib.swiglu_gate_up.restype = _I
lib.swiglu_ffn.argtypes = [_I, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
lib.swiglu_ffn.restype = _I
lib.swiglu_ffn_noalloc.argtypes = [_I, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]
lib.swiglu_ffn_noalloc.restype = _I
NOALLOC_SCRATCH_ELEMS = 1 << 23   # QG_NOALLOC_SCRATCH_ELEMS of include/qgemv.h
lib.swiglu_ffn_scratch_elems.argtypes = [_I, _I64, _I64, _I64]
lib.swiglu_ffn_scratch_elems.restype = _I64
lib.swiglu_ffn_block.argtypes = [_I, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
lib.swiglu_ffn_block.restype = _I
lib.swiglu_ffn_block_scratch_elems.argtypes = [_I, _I64, _I64, _I64]
lib.swiglu_ffn_block_scratch_elems.restype = _I64
lib.qgemv_argmax.argtypes = [_P, _P, _I64, _I64, _P]
lib.qgemv_argmax.restype = _I
lib.qgemv_head_argmax.argtypes = [_I, _P, _P, _P, _P, _I64, _I64, _I64, _P]
lib.qgemv_head_argmax.restype = _I
lib.qgemv_head_argmax_ws.argtypes = [_I, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P]
lib.qgemv_head_argmax_ws.restype = _I
lib.qgemv_head_argmax_workspace_bytes.argtypes = [_I, _I64, _I64]
lib.qgemv_head_argmax_workspace_bytes.restype = _I64
lib.qdequant.argtypes = [_I, _P, _P, _I64, _I64, _P]
lib.qdequant.restype = _I
lib.qgemv_q8act.argtypes = [_I, _P, _P, _P, _I64, _I64, _I64, _P]
lib.qgemv_q8act.restype = _I
lib.swiglu_ffn_q8act.argtypes = [_I, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
lib.swiglu_ffn_q8act.restype = _I
lib.swiglu_ffn_q8act_scratch_elems.argtypes = [_I, _I64, _I64, _I64]
lib.swiglu_ffn_q8act_scratch_elems.restype = _I64
lib.qgemv_q8act_ws.argtypes = [_I, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P]
lib.qgemv_q8act_ws.restype = _I
lib.qgemv_q8act_workspace_bytes.argtypes = [_I, _I64, _I64, _I64]
lib.qgemv_q8act_workspace_bytes.restype = _I64
lib.qquantize_q8_0.argtypes = [_P, _P, _I64, _I64, _P]
lib.qquantize_q8_0.restype = _I
lib.qgemv_set_launch_override.argtypes = [_I, _I, _I, _I, _I, _I]
lib.qgemv_set_launch_override.restype = _I
lib.qgemv_set_prefill_override.argtypes = [_I, _I, _I, _I, _I]
lib.qgemv_set_prefill_override.restype = _I
lib.qgemv_set_xs_override.argtypes = [_I, _I, _I, _I, _I, _I, _I]
lib.qgemv_set_xs_override.restype = _I
lib.qgemv_set_ffn_khalf.argtypes = [_I]
lib.qgemv_set_ffn_khalf.restype = _I
lib.qgemv_read_probe.argtypes = [_P, _I64, _I, _I, _P, _P]
lib.qgemv_read_probe.restype = _I
lib.qgemv_time_next_launch.argtypes = [_P, _P]
lib.qgemv_time_next_launch.restype = _I


class QGemvError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = int(status)
        msg = lib.qgemv_status_string(self.status).decode()
        super().__init__(f"{what}: {msg} (status {self.status})")


def _check(st, what):
    if st != 0:
        raise QGemvError(st, what)


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return int(t)
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


F32, U8, I8, I32 = torch.float32, torch.uint8, torch.int8, torch.int32


def _arg(t, name, dtype, min_numel=0):
    """Refuse, before any C call, a tensor the kernels would misread: not a
    torch tensor, not on the GPU, not contiguous, of another element type, or
    with fewer elements than the call reads or writes."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.numel() < min_numel:
        raise ValueError(f"{name}: needs at least {min_numel} elements, has {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensors must be contiguous")


def _on_gpu(*ts):
    """After every argument's type and size checks: all of them on the GPU."""
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _ntok(x, cols, name="x"):
    """Tokens in an activation tensor x [n_tok][cols] (or [cols]); refuses a
    size that is not a whole number of rows of cols."""
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(x).__name__}")
    if cols < 1 or x.numel() < cols or x.numel() % cols:
        raise ValueError(f"{name}: {x.numel()} elements is not a whole number of rows of {cols}")
    return x.numel() // cols


def _packed(t, fmt, rows, cols, name="packed"):
    _arg(t, name, U8, packed_bytes(fmt, rows, cols))


def layout_version() -> int:
    return lib.qgemv_layout_version()


def max_cols() -> int:
    v = lib.qgemv_max_cols()
    if v < 0:
        raise QGemvError(v, "qgemv_max_cols")
    return v


def packed_bytes(fmt, rows, cols) -> int:
    v = lib.qgemv_packed_bytes(_fmt(fmt), rows, cols)
    if v < 0:
        raise QGemvError(v, "qgemv_packed_bytes")
    return v


def set_launch_override(lpr=0, r=0, waves=0, depth=2, max_wg=0, cpl=1):
    """Force a GEMV launch shape (tuning); lpr=0 restores the built-in choice."""
    _check(lib.qgemv_set_launch_override(lpr, r, waves, depth, max_wg, cpl), "qgemv_set_launch_override")


def set_xs_override(mode=0, rs=0, seg=0, depth=0, nrs=0, order=-1, wg_per_cu=-1):
    """Row-streaming one-token kernel: mode 0 built-in, -1 off (lane-group
    kernels), 1 forced with the given fields (0 / -1 = built-in value)."""
    _check(lib.qgemv_set_xs_override(mode, rs, seg, depth, nrs, order, wg_per_cu), "qgemv_set_xs_override")


def set_ffn_khalf(mode=0):
    """One-token Q4_0 SwiGLU block: its down product in K halves (atomic adds
    of two half-row sums onto a cleared output): 0 built-in, 1 off, 2 on."""
    _check(lib.qgemv_set_ffn_khalf(mode), "qgemv_set_ffn_khalf")


def prefill_plan(fmt, nmat, rows, cols, n_tok, part_elems=0, cus=256):
    """(mtr, ntw, waves, run, ksplit): the matrix-core tile and K split of one product (host only)."""
    plan = (ctypes.c_int * 5)()
    _check(lib.qgemv_prefill_plan(_fmt(fmt), nmat, rows, cols, n_tok, part_elems, cus, plan), "qgemv_prefill_plan")
    return tuple(plan)


def set_prefill_override(mtr=0, ntw=0, waves=0, run=0, ksplit=0):
    """Force the matrix-core tile shape (n_tok > 1); mtr=0 restores the
    built-in choice, mtr=-1 turns the matrix-core path off (per-token GEMV)."""
    if mtr > 0 and run == 0:
        run = 1
    _check(lib.qgemv_set_prefill_override(mtr, ntw, waves, run, ksplit), "qgemv_set_prefill_override")


# ------------------------------------------------------------- repack ------

def _raw_bytes(fmt, rows, cols):
    """Bytes of the raw blocks of a [rows][cols] tensor (the layouts in qgemv.h)."""
    f = _fmt(fmt)
    per = {0: (32, 18), 1: (32, 34), 2: (256, 144), 4: (256, 210), 3: (1, 1)}[f]
    return rows * (cols // per[0]) * per[1]


def qgemv_repack_q4_0(raw, packed, rows, cols, stream=None):
    _arg(raw, "raw", U8, _raw_bytes(0, rows, cols))
    _packed(packed, 0, rows, cols)
    _on_gpu(raw, packed)
    _check(lib.qgemv_repack_q4_0(_ptr(raw), _ptr(packed), rows, cols, _stream(stream)), "qgemv_repack_q4_0")


def qgemv_repack_q8_0(raw, packed, rows, cols, stream=None):
    _arg(raw, "raw", U8, _raw_bytes(1, rows, cols))
    _packed(packed, 1, rows, cols)
    _on_gpu(raw, packed)
    _check(lib.qgemv_repack_q8_0(_ptr(raw), _ptr(packed), rows, cols, _stream(stream)), "qgemv_repack_q8_0")


def qgemv_repack_q4_k(raw, packed, rows, cols, stream=None):
    _arg(raw, "raw", U8, _raw_bytes(2, rows, cols))
    _packed(packed, 2, rows, cols)
    _on_gpu(raw, packed)
    _check(lib.qgemv_repack_q4_k(_ptr(raw), _ptr(packed), rows, cols, _stream(stream)), "qgemv_repack_q4_k")


def qgemv_repack_q6_k(raw, packed, rows, cols, stream=None):
    _arg(raw, "raw", U8, _raw_bytes(4, rows, cols))
    _packed(packed, 4, rows, cols)
    _on_gpu(raw, packed)
    _check(lib.qgemv_repack_q6_k(_ptr(raw), _ptr(packed), rows, cols, _stream(stream)), "qgemv_repack_q6_k")


def qgemv_repack_i8row(q, row_scale, packed, rows, cols, stream=None):
    _arg(q, "q", I8, rows * cols)
    _arg(row_scale, "row_scale", F32, rows)
    _packed(packed, 3, rows, cols)
    _on_gpu(q, row_scale, packed)
    _check(lib.qgemv_repack_i8row(_ptr(q), _ptr(row_scale), _ptr(packed), rows, cols, _stream(stream)),
           "qgemv_repack_i8row")


def repack(fmt, raw, rows, cols, row_scale=None, stream=None) -> torch.Tensor:
    """Allocate (torch) and fill a packed buffer from raw blocks on the GPU."""
    f = _fmt(fmt)
    nbytes = packed_bytes(f, rows, cols)
    dev = raw.device
    packed = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    off = (-packed.data_ptr()) % 256
    packed = packed[off:off + nbytes]
    if f == 0:
        qgemv_repack_q4_0(raw, packed, rows, cols, stream)
    elif f == 1:
        qgemv_repack_q8_0(raw, packed, rows, cols, stream)
    elif f == 2:
        qgemv_repack_q4_k(raw, packed, rows, cols, stream)
    elif f == 4:
        qgemv_repack_q6_k(raw, packed, rows, cols, stream)
    else:
        qgemv_repack_i8row(raw, row_scale, packed, rows, cols, stream)
    return packed


# ------------------------------------------------------------- products ----
def _y(y, shape, dev):
    if y is None:
        return torch.empty(shape, dtype=torch.float32, device=dev)
    return y


def qgemv(fmt, packed, x, rows, cols, y=None, stream=None) -> torch.Tensor:
    """y [n_tok][rows] = W x, x fp32 [n_tok][cols] (or [cols])."""
    n_tok = _ntok(x, cols)
    y = _y(y, (rows,) if x.dim() == 1 else (n_tok, rows), x.device)
    _packed(packed, fmt, rows, cols)
    _arg(x, "x", F32)
    _arg(y, "y", F32, n_tok * rows)
    _on_gpu(packed, x, y)
    _check(lib.qgemv(_fmt(fmt), _ptr(packed), _ptr(x), _ptr(y), rows, cols, n_tok, _stream(stream)), "qgemv")
    return y


def _gemv_named(name, fmtid):
    cfn = getattr(lib, name)

    def f(packed, x, y, rows, cols, n_tok=1, stream=None):
        _packed(packed, fmtid, rows, cols)
        _arg(x, "x", F32, n_tok * cols)
        _arg(y, "y", F32, n_tok * rows)
        _on_gpu(packed, x, y)
        _check(cfn(_ptr(packed), _ptr(x), _ptr(y), rows, cols, n_tok, _stream(stream)), name)
        return y
    f.__name__ = name
    f.__doc__ = f"Binding of {name}(packed, x, y, rows, cols, n_tok, stream)."
    return f


qgemv_q4_0 = _gemv_named("qgemv_q4_0", 0)
qgemv_q8_0 = _gemv_named("qgemv_q8_0", 1)
qgemv_q4_k = _gemv_named("qgemv_q4_k", 2)
qgemv_i8row = _gemv_named("qgemv_i8row", 3)
qgemv_q6_k = _gemv_named("qgemv_q6_k", 4)


def swiglu_gate_up(fmt, wg, wu, x, d_model, ffn, h=None, stream=None) -> torch.Tensor:
    n_tok = _ntok(x, d_model)
    h = _y(h, (n_tok, ffn), x.device)
    _packed(wg, fmt, ffn, d_model, "wg")
    _packed(wu, fmt, ffn, d_model, "wu")
    _arg(x, "x", F32)
    _arg(h, "h", F32, n_tok * ffn)
    _on_gpu(wg, wu, x, h)
    _check(lib.swiglu_gate_up(_fmt(fmt), _ptr(wg), _ptr(wu), _ptr(x), _ptr(h), d_model, ffn, n_tok,
                              _stream(stream)), "swiglu_gate_up")
    return h


def _ffn_args(fmt, wg, wu, wd, x, out, h_scratch, d_model, ffn, n_tok):
    _packed(wg, fmt, ffn, d_model, "wg")
    _packed(wu, fmt, ffn, d_model, "wu")
    _packed(wd, fmt, d_model, ffn, "wd")
    _arg(x, "x", F32)
    _arg(out, "out", F32, n_tok * d_model)
    _arg(h_scratch, "h_scratch", F32, n_tok * ffn)


def swiglu_ffn_scratch_elems(fmt, d_model, ffn, n_tok) -> int:
    v = lib.swiglu_ffn_scratch_elems(_fmt(fmt), d_model, ffn, n_tok)
    _check(v if v < 0 else 0, "swiglu_ffn_scratch_elems")
    return v


def swiglu_ffn(fmt, wg, wu, wd, x, d_model, ffn, out=None, h_scratch=None, stream=None):
    """(out, h): out [n_tok][d_model] = Wd (silu(Wg x) * (Wu x)); h [n_tok][ffn]
    is a view of the scratch (allocated at swiglu_ffn_scratch_elems if None)."""
    n_tok = _ntok(x, d_model)
    out = _y(out, (n_tok, d_model), x.device)
    if h_scratch is None:
        h_scratch = torch.empty(swiglu_ffn_scratch_elems(fmt, d_model, ffn, n_tok), dtype=torch.float32,
                                device=x.device)
    _ffn_args(fmt, wg, wu, wd, x, out, h_scratch, d_model, ffn, n_tok)
    _on_gpu(wg, wu, wd, x, out, h_scratch)
    _check(lib.swiglu_ffn(_fmt(fmt), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(x), _ptr(out), _ptr(h_scratch),
                          h_scratch.numel(), d_model, ffn, n_tok, _stream(stream)), "swiglu_ffn")
    return out, h_scratch.view(-1)[:n_tok * ffn].view(n_tok, ffn)


def swiglu_ffn_noalloc(fmt, wg, wu, wd, x, d_model, ffn, out=None, stream=None) -> torch.Tensor:
    """out [n_tok][d_model] = Wd (silu(Wg x) * (Wu x)) with the library's own
    per-device scratch (no allocation in the call; calls overlapping on one
    device race)."""
    n_tok = _ntok(x, d_model)
    out = _y(out, (n_tok, d_model), x.device)
    _packed(wg, fmt, ffn, d_model, "wg")
    _packed(wu, fmt, ffn, d_model, "wu")
    _packed(wd, fmt, d_model, ffn, "wd")
    _arg(x, "x", F32)
    _arg(out, "out", F32, n_tok * d_model)
    _on_gpu(wg, wu, wd, x, out)
    _check(lib.swiglu_ffn_noalloc(_fmt(fmt), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(x), _ptr(out), d_model, ffn, n_tok,
                                  _stream(stream)), "swiglu_ffn_noalloc")
    return out


def q8act_workspace_bytes(fmt, rows, cols, n_tok) -> int:
    """Bytes of workspace for the batched Q8_0-activation product (host only)."""
    n = lib.qgemv_q8act_workspace_bytes(_fmt(fmt), rows, cols, n_tok)
    _check(n if n < 0 else 0, "qgemv_q8act_workspace_bytes")
    return n


def qgemv_q8act(fmt, packed, x, rows, cols, y=None, workspace=None, stream=None) -> torch.Tensor:
    """y [n_tok][rows] = W xq, xq the Q8_0 representation of x (Q4_0, Q8_0
    weights).  Several tokens: the batched launches, with workspace (uint8, at
    least the quantized activations' bytes; q8act_workspace_bytes for the
    built-in K split; made when none is given)."""
    n_tok = _ntok(x, cols)
    y = _y(y, (rows,) if x.dim() == 1 else (n_tok, rows), x.device)
    _packed(packed, fmt, rows, cols)
    _arg(x, "x", F32)
    _arg(y, "y", F32, n_tok * rows)
    if n_tok == 1:
        _on_gpu(packed, x, y)
        _check(lib.qgemv_q8act(_fmt(fmt), _ptr(packed), _ptr(x), _ptr(y), rows, cols, n_tok, _stream(stream)),
               "qgemv_q8act")
        return y
    if workspace is None:
        workspace = torch.empty(q8act_workspace_bytes(fmt, rows, cols, n_tok), dtype=torch.uint8, device=x.device)
    _arg(workspace, "workspace", torch.uint8)
    _on_gpu(packed, x, y, workspace)
    _check(lib.qgemv_q8act_ws(_fmt(fmt), _ptr(packed), _ptr(x), _ptr(y), rows, cols, n_tok, _ptr(workspace),
                              workspace.numel(), _stream(stream)), "qgemv_q8act_ws")
    return y


def swiglu_ffn_q8act_scratch_elems(fmt, d_model, ffn, n_tok) -> int:
    v = lib.swiglu_ffn_q8act_scratch_elems(_fmt(fmt), d_model, ffn, n_tok)
    _check(v if v < 0 else 0, "swiglu_ffn_q8act_scratch_elems")
    return v


def swiglu_ffn_q8act(fmt, wg, wu, wd, x, d_model, ffn, out=None, h_scratch=None, stream=None):
    """(out, h): the SwiGLU FFN with x and h quantized to Q8_0 before their
    products; h_scratch made with swiglu_ffn_q8act_scratch_elems floats (the
    batched path for several tokens) when none is given."""
    n_tok = _ntok(x, d_model)
    out = _y(out, (n_tok, d_model), x.device)
    if h_scratch is None:
        h_scratch = torch.empty(swiglu_ffn_q8act_scratch_elems(fmt, d_model, ffn, n_tok), dtype=torch.float32,
                                device=x.device)
    _ffn_args(fmt, wg, wu, wd, x, out, h_scratch, d_model, ffn, n_tok)
    _on_gpu(wg, wu, wd, x, out, h_scratch)
    _check(lib.swiglu_ffn_q8act(_fmt(fmt), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(x), _ptr(out), _ptr(h_scratch),
                                h_scratch.numel(), d_model, ffn, n_tok, _stream(stream)), "swiglu_ffn_q8act")
    return out, h_scratch.view(-1)[:n_tok * ffn].view(n_tok, ffn)


def qquantize_q8_0(x, n, blocks=None, stream=None) -> torch.Tensor:
    """Raw Q8_0 blocks (uint8 [n_tok][n/32 * 34]) of activation rows x [n_tok][n]."""
    n_tok = _ntok(x, n)
    if blocks is None:
        blocks = torch.empty((n_tok, n // 32 * 34), dtype=torch.uint8, device=x.device)
    _arg(x, "x", F32)
    _arg(blocks, "blocks", U8, n_tok * (n // 32) * 34)
    _on_gpu(x, blocks)
    _check(lib.qquantize_q8_0(_ptr(x), _ptr(blocks), n, n_tok, _stream(stream)), "qquantize_q8_0")
    return blocks


def qdequant(fmt, packed, rows, cols, w_out=None, stream=None) -> torch.Tensor:
    _packed(packed, fmt, rows, cols)
    w_out = _y(w_out, (rows, cols), packed.device)
    _arg(w_out, "w_out", F32, rows * cols)
    _on_gpu(packed, w_out)
    _check(lib.qdequant(_fmt(fmt), _ptr(packed), _ptr(w_out), rows, cols, _stream(stream)), "qdequant")
    return w_out


def swiglu_ffn_block_scratch_elems(fmt, d_model, ffn, n_tok) -> int:
    v = lib.swiglu_ffn_block_scratch_elems(_fmt(fmt), d_model, ffn, n_tok)
    _check(v if v < 0 else 0, "swiglu_ffn_block_scratch_elems")
    return v


def swiglu_ffn_block(fmt, wg, wu, wd, gamma, eps, x, d_model, ffn, out=None, h_scratch=None, stream=None):
    """(out, h): out = x + Wd (silu(Wg xn) * (Wu xn)), xn = rmsnorm(x) * gamma; out may be x
    (in place).  h [n_tok][ffn] is a view of the scratch (allocated at
    swiglu_ffn_block_scratch_elems if None)."""
    n_tok = _ntok(x, d_model)
    out = _y(out, (n_tok, d_model), x.device)
    if h_scratch is None:
        h_scratch = torch.empty(swiglu_ffn_block_scratch_elems(fmt, d_model, ffn, n_tok), dtype=torch.float32,
                                device=x.device)
    _ffn_args(fmt, wg, wu, wd, x, out, h_scratch, d_model, ffn, n_tok)
    _arg(gamma, "gamma", F32, d_model)
    _on_gpu(wg, wu, wd, gamma, x, out, h_scratch)
    _check(lib.swiglu_ffn_block(_fmt(fmt), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(gamma), float(eps), _ptr(x), _ptr(out),
                                _ptr(h_scratch), h_scratch.numel(), d_model, ffn, n_tok, _stream(stream)),
           "swiglu_ffn_block")
    return out, h_scratch.view(-1)[:n_tok * ffn].view(n_tok, ffn)


def qgemv_argmax(logits, n, token=None, stream=None) -> torch.Tensor:
    """int32 [n_tok]: first index of the largest logit of each row of logits [n_tok][n]."""
    n_tok = _ntok(logits, n, "logits")
    if token is None:
        token = torch.empty(n_tok, dtype=torch.int32, device=logits.device)
    _arg(logits, "logits", F32)
    _arg(token, "token", I32, n_tok)
    _on_gpu(logits, token)
    _check(lib.qgemv_argmax(_ptr(logits), _ptr(token), n, n_tok, _stream(stream)), "qgemv_argmax")
    return token


def head_argmax_workspace_bytes(fmt, rows, cols):
    """Bytes of workspace the fused head needs (host only)."""
    n = lib.qgemv_head_argmax_workspace_bytes(_fmt(fmt), rows, cols)
    _check(n if n < 0 else 0, "qgemv_head_argmax_workspace_bytes")
    return n


def qgemv_head_argmax(fmt, packed, x, rows, cols, logits=None, token=None, workspace=None, fused=False, stream=None):
    """(token int32 [n_tok], logits [n_tok][rows]): the head product and greedy
    sampling: the product, then the argmax launch over the logits; or (fused,
    one token) the product writing one candidate per workgroup into workspace
    (uint8, at least head_argmax_workspace_bytes; made when none is given),
    then a one-workgroup launch combining them."""
    n_tok = _ntok(x, cols)
    logits = _y(logits, (n_tok, rows), x.device)
    if token is None:
        token = torch.empty(n_tok, dtype=torch.int32, device=x.device)
    _packed(packed, fmt, rows, cols)
    _arg(x, "x", F32)
    _arg(logits, "logits", F32, n_tok * rows)
    _arg(token, "token", I32, n_tok)
    if not fused:
        _on_gpu(packed, x, logits, token)
        _check(lib.qgemv_head_argmax(_fmt(fmt), _ptr(packed), _ptr(x), _ptr(logits), _ptr(token), rows, cols, n_tok,
                                     _stream(stream)), "qgemv_head_argmax")
        return token, logits
    need = head_argmax_workspace_bytes(fmt, rows, cols)
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
    _arg(workspace, "workspace", U8, need)
    _on_gpu(packed, x, logits, token, workspace)
    _check(lib.qgemv_head_argmax_ws(_fmt(fmt), _ptr(packed), _ptr(x), _ptr(logits), _ptr(token), rows, cols, n_tok,
                                    _ptr(workspace), workspace.numel(), _stream(stream)), "qgemv_head_argmax_ws")
    return token, logits
