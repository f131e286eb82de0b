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
