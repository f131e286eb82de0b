"""The measurement hook qgemv_time_next_launch: the next GEMV launch carries
the caller's start/stop events (hipExtLaunchKernel), its results are those of
an ordinary launch, and the events time that one kernel."""
import ctypes

import numpy as np
import pytest

import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def test_timed_launch_same_result_and_positive_time():
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    ev = [ctypes.c_void_p() for _ in range(2)]
    for e in ev:
        assert hip.hipEventCreateWithFlags(ctypes.byref(e), 0) == 0
    try:
        rng = np.random.default_rng(4000)
        t = synth.make_tensor("q4_0", 4096, 5120, rng)
        pk = G.upload(t)
        x = rng.standard_normal(5120).astype(np.float32)
        y0 = G.gemv_gpu(t, pk, x)
        assert G.qg().lib.qgemv_time_next_launch(ev[0], ev[1]) == 0
        y1 = G.gemv_gpu(t, pk, x)
        assert hip.hipEventSynchronize(ev[1]) == 0
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
        assert np.array_equal(y0, y1)
        assert 0.0 < ms.value < 1000.0
        # consumed by that launch: the next one runs untimed
        assert np.array_equal(G.gemv_gpu(t, pk, x), y0)
    finally:
        for e in ev:
            hip.hipEventDestroy(e)


def test_two_queued_pairs_time_both_ffn_kernels():
    # two pairs queued before one swiglu_ffn call: the first times its gate/up
    # launch, the second its down launch (K halves on this shape); the results
    # are those of an untimed call
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    ev = [ctypes.c_void_p() for _ in range(4)]
    for e in ev:
        assert hip.hipEventCreateWithFlags(ctypes.byref(e), 0) == 0
    try:
        d_model, ffn = 5120, 17408
        rng = np.random.default_rng(4001)
        tens = [synth.make_tensor("q4_0", ffn, d_model, rng), synth.make_tensor("q4_0", ffn, d_model, rng),
                synth.make_tensor("q4_0", d_model, ffn, rng)]
        pk = [G.upload(t) for t in tens]
        xd = G.torch.from_numpy(rng.standard_normal((1, d_model)).astype(np.float32)).to(G.dev())

        def run():
            out, h = G.qg().swiglu_ffn("q4_0", pk[0], pk[1], pk[2], xd, d_model, ffn)
            G.torch.cuda.synchronize()
            return out.cpu().numpy(), h.cpu().numpy()

        o0, h0 = run()
        assert G.qg().lib.qgemv_time_next_launch(ev[0], ev[1]) == 0
        assert G.qg().lib.qgemv_time_next_launch(ev[2], ev[3]) == 0
        o1, h1 = run()
        ms = []
        for a, b in ((0, 1), (2, 3)):
            assert hip.hipEventSynchronize(ev[b]) == 0
            m = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(m), ev[a], ev[b]) == 0
            ms.append(m.value)
        assert np.array_equal(o0, o1) and np.array_equal(h0, h1)
        assert all(0.0 < m < 1000.0 for m in ms)
        # the down product starts after the gate/up product ends
        gap = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(gap), ev[1], ev[2]) == 0
        assert gap.value >= 0.0
        # both pairs consumed: the next call runs untimed
        o2, _ = run()
        assert np.array_equal(o2, o0)
    finally:
        for e in ev:
            hip.hipEventDestroy(e)
