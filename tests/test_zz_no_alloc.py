"""swiglu_ffn_noalloc (the allocation-free variant of swiglu_ffn, scratch in
the library's per-device array) through the C ABI against swiglu_ffn given the
same amount of caller scratch: bit-identical outputs, on two calls in a row
(the second smaller, after the first left its contents in the shared array),
both repeated; and its refusals."""
import ctypes

import numpy as np
import pytest

import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _ffn(fmt, d_model, ffn, seed):
    rng = np.random.default_rng(seed)
    tens = [synth.make_tensor(fmt, ffn, d_model, rng), synth.make_tensor(fmt, ffn, d_model, rng),
            synth.make_tensor(fmt, d_model, ffn, rng)]
    return [G.upload(t) for t in tens], rng


def _both(fmt, pk, x, d_model, ffn):
    torch = G.torch
    qg = G.qg()
    n_tok = x.shape[0]
    lib = qg.lib
    s = torch.cuda.current_stream().cuda_stream
    out_a = torch.full((n_tok, d_model), float("nan"), device=G.dev())
    st = lib.swiglu_ffn_noalloc(qg.FORMATS[fmt], pk[0].data_ptr(), pk[1].data_ptr(), pk[2].data_ptr(), x.data_ptr(),
                                out_a.data_ptr(), d_model, ffn, n_tok, s)
    assert st == 0, st
    elems = min(qg.swiglu_ffn_scratch_elems(fmt, d_model, ffn, n_tok), qg.NOALLOC_SCRATCH_ELEMS)
    sc = torch.full((elems,), float("nan"), device=G.dev())
    out_b, _ = qg.swiglu_ffn(fmt, pk[0], pk[1], pk[2], x, d_model, ffn, h_scratch=sc)
    torch.cuda.synchronize()
    return out_a.cpu().numpy(), out_b.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    (("q4_0", 5120, 17408, 8), ("q4_0", 576, 1536, 1)),      # matrix cores, split K, bf16 copies; then one token
    (("i8row", 2048, 8192, 128), ("q4_k", 2048, 5632, 5)),   # 128 tokens; then a smaller matrix-core product
    (("q4_0", 5120, 17408, 1), ("q8_0", 288, 768, 3)),       # the one-token FFN; then 3 tokens
])
def test_noalloc_matches_swiglu_ffn_two_calls(first, second):
    runs = []
    for k, (fmt, d_model, ffn, n_tok) in enumerate((first, second)):
        pk, rng = _ffn(fmt, d_model, ffn, 5000 + 7 * k + d_model)
        x = G.torch.from_numpy(rng.standard_normal((n_tok, d_model)).astype(np.float32)).to(G.dev())
        runs.append((fmt, pk, x, d_model, ffn))
    for fmt, pk, x, d_model, ffn in runs + runs:   # in a row, then again
        a, b = _both(fmt, pk, x, d_model, ffn)
        assert np.all(np.isfinite(a))
        assert np.array_equal(a, b), (fmt, d_model, ffn, x.shape[0])


def test_noalloc_refusals():
    lib = G.qg().lib
    null = ctypes.c_void_p(0)
    # h alone would not fit the array: refused before any device work
    assert lib.swiglu_ffn_noalloc(0, null, null, null, null, null, 5120, 17408, 482, null) == -6
    assert lib.swiglu_ffn_noalloc(9, null, null, null, null, null, 64, 64, 1, null) == -4
    assert lib.swiglu_ffn_noalloc(0, null, null, null, null, null, 64, 48, 1, null) == -2
    pk, rng = _ffn("q4_0", 256, 512, 5100)
    x = G.torch.zeros((1, 256), device=G.dev())
    assert lib.swiglu_ffn_noalloc(0, pk[0].data_ptr(), pk[1].data_ptr(), pk[2].data_ptr(), x.data_ptr(), null,
                                  256, 512, 1, null) == -1
    assert lib.swiglu_ffn_noalloc(0, pk[0].data_ptr(), pk[1].data_ptr(), pk[2].data_ptr(), x.data_ptr(),
                                  x.data_ptr(), 256, 512, 1, null) == -5   # out overlaps x
