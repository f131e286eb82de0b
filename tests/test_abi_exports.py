"""The C-ABI library loads and exports every function include/qgemv.h declares.

CPU only: nothing here launches a kernel or queries a device; the refusal
checks exercised return before any HIP call (format, null pointer and shape
are validated first).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "dequant_matrix_vector_amd", "libqgemv.so")
HEADER = os.path.join(ROOT, "include", "qgemv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libqgemv.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("qgemv_q4_0", "qgemv_q8_0", "qgemv_q4_k", "qgemv_i8row", "swiglu_ffn", "qdequant",
              "qgemv_repack_q4_0", "qgemv_repack_q8_0", "qgemv_repack_q4_k", "qgemv_repack_i8row",
              "qgemv_packed_bytes", "qgemv_status_string"):
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_host_only_queries(lib):
    lib.qgemv_packed_bytes.restype = ctypes.c_int64
    lib.qgemv_packed_bytes.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
    # quant plane padded to 256 B, then the scale plane, padded to 256 B
    assert lib.qgemv_packed_bytes(0, 17408, 5120) == 17408 * 2560 + 17408 * 160 * 2
    assert lib.qgemv_packed_bytes(1, 49152, 576) == 49152 * 576 + 49152 * 18 * 2
    assert lib.qgemv_packed_bytes(2, 3, 256) == 512 + 256
    assert lib.qgemv_packed_bytes(3, 5, 32) == 256 + 256
    # Q6_K: low-nibble, high-bit, scale and d planes; 210 bytes per 256 weights
    assert lib.qgemv_packed_bytes(4, 32000, 2048) == 32000 * 8 * 210
    assert lib.qgemv_packed_bytes(4, 3, 256) == 512 + 256 + 256 + 256
    assert lib.qgemv_packed_bytes(4, 3, 288) == -2
    assert lib.qgemv_packed_bytes(0, 4, 48) == -2     # not a block multiple
    assert lib.qgemv_packed_bytes(9, 4, 64) == -4     # unknown format
    lib.qgemv_status_string.restype = ctypes.c_char_p
    assert lib.qgemv_status_string(0) == b"ok"
    assert b"shape" in lib.qgemv_status_string(-2)
    assert lib.qgemv_layout_version() == 1


def test_refusals_before_any_device_call(lib):
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.qgemv.argtypes = [ctypes.c_int, P, P, P, I64, I64, I64, P]
    fake = ctypes.c_void_p(0x100000)
    assert lib.qgemv(7, fake, fake, fake, 4, 32, 1, None) == -4
    assert lib.qgemv(0, None, fake, fake, 4, 32, 1, None) == -1
    assert lib.qgemv(0, fake, fake, fake, 4, 33, 1, None) == -2
    assert lib.qgemv(0, fake, fake, fake, 0, 32, 1, None) == -2
    assert lib.qgemv(0, fake, fake, fake, 4, 32, 0, None) == -2
    assert lib.qgemv(2, fake, fake, fake, 4, 300, 1, None) == -2
    assert lib.qgemv(4, fake, fake, fake, 4, 288, 1, None) == -2
    # Q8_0 activations: Q4_0 and Q8_0 weights only; the quantizer's shape rules
    lib.qgemv_q8act.argtypes = [ctypes.c_int, P, P, P, I64, I64, I64, P]
    assert lib.qgemv_q8act(2, fake, fake, fake, 4, 256, 1, None) == -4
    assert lib.qgemv_q8act(4, fake, fake, fake, 4, 256, 1, None) == -4
    lib.qgemv_q8act_ws.argtypes = [ctypes.c_int, P, P, P, I64, I64, I64, P, I64, P]
    assert lib.qgemv_q8act_ws(2, fake, fake, fake, 4, 256, 8, fake, 1 << 20, None) == -4
    lib.qgemv_q8act_workspace_bytes.argtypes = [ctypes.c_int, I64, I64, I64]
    lib.qgemv_q8act_workspace_bytes.restype = I64
    lib.swiglu_ffn_q8act_scratch_elems.argtypes = [ctypes.c_int, I64, I64, I64]
    lib.swiglu_ffn_q8act_scratch_elems.restype = I64
    # host-only sizes: one token needs no workspace; several need at least the
    # quantized activations (64 + 4 bytes per block)
    assert lib.qgemv_q8act_workspace_bytes(0, 100, 256, 1) == 0
    assert lib.qgemv_q8act_workspace_bytes(0, 100, 256, 8) >= 8 * 8 * 68
    assert lib.qgemv_q8act_workspace_bytes(2, 100, 256, 8) == -4
    assert lib.qgemv_q8act_workspace_bytes(0, 100, 250, 8) == -2
    assert lib.swiglu_ffn_q8act_scratch_elems(0, 576, 1536, 1) == 1536
    assert lib.swiglu_ffn_q8act_scratch_elems(1, 576, 1536, 8) >= 8 * 1536 + 8 * 48 * 68 // 4
    lib.qquantize_q8_0.argtypes = [P, P, I64, I64, P]
    assert lib.qquantize_q8_0(fake, fake, 48, 1, None) == -2
    assert lib.qquantize_q8_0(fake, fake, 64, 0, None) == -2
    assert lib.qquantize_q8_0(None, fake, 64, 1, None) == -1
    # the timing hook wants both events or neither
    lib.qgemv_time_next_launch.argtypes = [P, P]
    assert lib.qgemv_time_next_launch(fake, None) == -1
    assert lib.qgemv_time_next_launch(None, None) == 0
    # a queue of at most four pairs (nothing is launched, so nothing is
    # recorded into the placeholder handles); NULL, NULL empties it
    for _ in range(4):
        assert lib.qgemv_time_next_launch(fake, fake) == 0
    assert lib.qgemv_time_next_launch(fake, fake) == -2
    assert lib.qgemv_time_next_launch(None, None) == 0
    assert lib.qgemv_time_next_launch(fake, fake) == 0
    assert lib.qgemv_time_next_launch(None, None) == 0


def test_prefill_override_validation(lib):
    # host-only: the tile-shape hook validates its arguments without a device
    f = lib.qgemv_set_prefill_override
    f.argtypes = [ctypes.c_int] * 5
    f.restype = ctypes.c_int
    for bad in ((3, 1, 4, 2, 0), (1, 3, 4, 2, 0), (1, 1, 2, 2, 0), (2, 16, 8, 2, 0), (1, 1, 4, 3, 0),
                (1, 1, 4, 8, 0), (1, 1, 4, 2, -1), (1, 1, 4, 2, 65)):
        assert f(*bad) == -2, bad
    assert f(2, 8, 4, 2, 0) == 0 and f(1, 2, 8, 4, 3) == 0 and f(1, 1, 8, 1, 0) == 0 and f(-1, 0, 0, 0, 0) == 0
    assert f(0, 0, 0, 0, 0) == 0


def test_prefill_plan_pins_the_tile_rules(lib):
    # host only: the tile and K split the matrix-core path picks, for 256 CUs,
    # on the shapes its rules were measured on (per-kernel traces at 8, 64
    # and 128 tokens); room = partial-sum floats the call gives
    I64 = ctypes.c_int64
    f = lib.qgemv_prefill_plan
    f.argtypes = [ctypes.c_int, ctypes.c_int, I64, I64, I64, I64, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    f.restype = ctypes.c_int
    lib.qgemv_set_prefill_override.argtypes = [ctypes.c_int] * 5
    assert lib.qgemv_set_prefill_override(0, 0, 0, 0, 0) == 0

    def plan(fmt, nmat, rows, cols, n_tok, room):
        out = (ctypes.c_int * 5)()
        assert f(fmt, nmat, rows, cols, n_tok, room, 256, out) == 0
        return tuple(out)

    big = 1 << 40
    # 27B-class FFN (swiglu_ffn, K split allowed): the pair and the down product
    assert plan(0, 2, 17408, 5120, 128, big) == (1, 8, 8, 1, 1)
    assert plan(0, 1, 5120, 17408, 128, big) == (1, 4, 8, 1, 4)
    assert plan(0, 2, 17408, 5120, 64, big) == (1, 4, 4, 1, 2)
    assert plan(0, 2, 17408, 5120, 8, big) == (1, 1, 4, 2, 4)
    assert plan(0, 1, 5120, 17408, 8, big) == (1, 1, 4, 2, 12)
    assert plan(3, 1, 2048, 8192, 128, big) == (1, 4, 8, 1, 8)
    # qgemv (no room): 2048-row products fall back to one token tile, long rows
    # with runs of four; tall heads keep 8 or 4 token tiles
    assert plan(4, 1, 2048, 5632, 128, 0) == (1, 1, 4, 4, 1)
    assert plan(2, 1, 2048, 2048, 128, 0) == (1, 1, 4, 2, 1)
    assert plan(3, 1, 49152, 2048, 128, 0) == (1, 8, 16, 1, 1)
    assert plan(4, 1, 32000, 2048, 128, 0) == (1, 4, 8, 1, 1)
    # the K split never exceeds the room given
    assert plan(0, 1, 5120, 17408, 8, 2 * 8 * 5120) == (1, 1, 4, 2, 2)
    # an override is honoured, a shape that is not built runs as the nearest built one
    assert lib.qgemv_set_prefill_override(2, 8, 16, 4, 1) == 0
    try:
        # the pair with 2 row tiles, 16 waves and runs of four is not built:
        # it runs as the nearest built shape, one row tile, 8 waves, runs of one
        assert plan(0, 2, 17408, 5120, 128, big) == (1, 8, 8, 1, 1)
    finally:
        assert lib.qgemv_set_prefill_override(0, 0, 0, 0, 0) == 0
    # refusals
    out = (ctypes.c_int * 5)(*([7] * 5))
    assert f(0, 1, 64, 64, 8, 0, 256, None) == -1
    assert f(9, 1, 64, 64, 8, 0, 256, out) == -4
    assert f(0, 3, 64, 64, 8, 0, 256, out) == -2
    assert f(0, 1, 64, 48, 8, 0, 256, out) == -2
    assert f(0, 1, 64, 64, 1, 0, 256, out) == -2
    assert f(0, 1, 64, 64, 8, 0, 0, out) == -2
    assert tuple(out) == (7,) * 5


def test_tuning_overrides_are_per_thread(lib):
    # a tuning override set on one thread leaves other threads' calls alone
    import threading
    I64 = ctypes.c_int64
    f = lib.qgemv_prefill_plan
    f.argtypes = [ctypes.c_int, ctypes.c_int, I64, I64, I64, I64, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    f.restype = ctypes.c_int
    lib.qgemv_set_prefill_override.argtypes = [ctypes.c_int] * 5
    lib.swiglu_ffn_scratch_elems.argtypes = [ctypes.c_int, I64, I64, I64]
    lib.swiglu_ffn_scratch_elems.restype = I64

    def plan():
        out = (ctypes.c_int * 5)()
        assert f(0, 2, 17408, 5120, 128, 1 << 40, 256, out) == 0
        return tuple(out)

    seen = {}

    def other():
        assert lib.qgemv_set_prefill_override(1, 4, 8, 1, 2) == 0
        seen["forced"] = plan()
        assert lib.qgemv_set_prefill_override(-1, 0, 0, 0, 0) == 0   # matrix cores off on this thread
        seen["scratch_off"] = lib.swiglu_ffn_scratch_elems(0, 5120, 17408, 8)
        assert lib.qgemv_set_prefill_override(0, 0, 0, 0, 0) == 0

    assert lib.qgemv_set_prefill_override(0, 0, 0, 0, 0) == 0
    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["forced"] == (1, 4, 8, 1, 2)
    assert seen["scratch_off"] == 8 * 17408
    assert plan() == (1, 8, 8, 1, 1)
    assert lib.swiglu_ffn_scratch_elems(0, 5120, 17408, 8) > 8 * 17408


def test_xs_override_refusals(lib):
    f = lib.qgemv_set_xs_override
    f.argtypes = [ctypes.c_int] * 7
    f.restype = ctypes.c_int
    assert f(2, 0, 0, 0, 0, -1, -1) == -2     # unknown mode
    assert f(1, -1, 0, 0, 0, -1, -1) == -2    # negative field
    assert f(1, 0, 0, 0, 0, 2, -1) == -2      # unknown order
    assert f(1, 0, 0, 0, 0, -1, 9) == -2      # too many workgroups per CU
    assert f(1, 2, 5, 2, 12, 1, 3) == 0
    assert f(-1, 0, 0, 0, 0, 0, 0) == 0
    assert f(0, 0, 0, 0, 0, 0, 0) == 0


def test_ffn_khalf_refusals(lib):
    f = lib.qgemv_set_ffn_khalf
    f.argtypes = [ctypes.c_int]
    f.restype = ctypes.c_int
    assert f(-1) == -2
    assert f(3) == -2
    for m in (2, 1, 0):
        assert f(m) == 0
