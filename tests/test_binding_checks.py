"""The Python binding refuses, before any C call, tensors the kernels would
misread: another element type, too few elements, an activation size that is
not a whole number of rows, a non-contiguous or host tensor.  CPU only: every
refusal below happens before the library is asked to touch device memory
(host tensors of the right type and size are refused last, for living on the
host)."""
import pytest
import torch

qg = pytest.importorskip("dequant_matrix_vector_amd")

F32, U8, I8, I32 = torch.float32, torch.uint8, torch.int8, torch.int32


def packed(fmt, rows, cols, extra=0, dtype=U8):
    return torch.zeros(qg.packed_bytes(fmt, rows, cols) + extra, dtype=dtype)


def refused(match, fn, *a, **k):
    with pytest.raises((ValueError, TypeError), match=match):
        fn(*a, **k)


R, C = 64, 256


def test_qgemv_refusals():
    pk, x, y = packed("q4_0", R, C), torch.zeros(C, dtype=F32), torch.zeros(R, dtype=F32)
    refused("expected torch.float32", qg.qgemv, "q4_0", pk, x.half(), R, C, y=y)
    refused("expected torch.float32", qg.qgemv, "q4_0", pk, x, R, C, y=y.double())
    refused("whole number of rows", qg.qgemv, "q4_0", pk, torch.zeros(C + 32, dtype=F32), R, C, y=y)
    refused("whole number of rows", qg.qgemv, "q4_0", pk, torch.zeros(C - 32, dtype=F32), R, C, y=y)
    refused("at least", qg.qgemv, "q4_0", pk, x, R, C, y=torch.zeros(R - 1, dtype=F32))
    refused("at least", qg.qgemv, "q4_0", pk, torch.zeros(2 * C, dtype=F32), R, C, y=y)   # 2 tokens, 1 row of y
    refused("at least", qg.qgemv, "q4_0", pk[:-1], x, R, C, y=y)
    refused("expected torch.uint8", qg.qgemv, "q4_0", packed("q4_0", R, C, dtype=I8), x, R, C, y=y)
    refused("contiguous", qg.qgemv, "q4_0", pk, torch.zeros(2 * C, dtype=F32)[::2], R, C, y=y)
    refused("expected a torch.Tensor", qg.qgemv, "q4_0", pk, [0.0] * C, R, C, y=y)
    refused("live on the GPU", qg.qgemv, "q4_0", pk, x, R, C, y=y)


def test_named_products_refusals():
    pk = packed("q8_0", R, C)
    refused("at least", qg.qgemv_q8_0, pk, torch.zeros(C, dtype=F32), torch.zeros(R, dtype=F32), R, C, n_tok=2)
    refused("expected torch.uint8", qg.qgemv_q4_k, packed("q4_k", R, C, dtype=I8), torch.zeros(C, dtype=F32),
            torch.zeros(R, dtype=F32), R, C)
    refused("at least", qg.qgemv_q6_k, packed("q6_k", R, C)[:-16], torch.zeros(C, dtype=F32),
            torch.zeros(R, dtype=F32), R, C)


def test_ffn_refusals():
    d, f = 256, 512
    wg, wu, wd = packed("q4_0", f, d), packed("q4_0", f, d), packed("q4_0", d, f)
    x, out = torch.zeros(d, dtype=F32), torch.zeros(d, dtype=F32)
    h = torch.zeros(f, dtype=F32)
    refused("h_scratch: expected torch.float32", qg.swiglu_ffn, "q4_0", wg, wu, wd, x, d, f, out=out,
            h_scratch=torch.zeros(f, dtype=torch.bfloat16))
    refused("h_scratch: needs at least", qg.swiglu_ffn, "q4_0", wg, wu, wd, x, d, f, out=out,
            h_scratch=torch.zeros(f - 1, dtype=F32))
    refused("wd: needs at least", qg.swiglu_ffn, "q4_0", wg, wu, packed("q4_0", f, d)[:100], x, d, f, out=out,
            h_scratch=h)
    refused("out: needs at least", qg.swiglu_ffn, "q4_0", wg, wu, wd, x, d, f, out=out[:-4], h_scratch=h)
    refused("whole number of rows", qg.swiglu_ffn, "q4_0", wg, wu, wd, torch.zeros(d + 1, dtype=F32), d, f,
            out=out, h_scratch=h)
    refused("gamma: needs at least", qg.swiglu_ffn_block, "q4_0", wg, wu, wd, torch.zeros(d - 4, dtype=F32),
            1e-5, x, d, f, out=out, h_scratch=h)
    refused("gamma: expected torch.float32", qg.swiglu_ffn_block, "q4_0", wg, wu, wd,
            torch.zeros(d, dtype=torch.float16), 1e-5, x, d, f, out=out, h_scratch=h)
    refused("h: needs at least", qg.swiglu_gate_up, "q4_0", wg, wu, x, d, f, h=h[:-1])
    refused("wu: expected torch.uint8", qg.swiglu_gate_up, "q4_0", wg, wu.view(torch.int8), x, d, f, h=h)
    refused("h_scratch: needs at least", qg.swiglu_ffn_q8act, "q4_0", wg, wu, wd, x, d, f, out=out,
            h_scratch=h[:-8])
    refused("live on the GPU", qg.swiglu_ffn, "q4_0", wg, wu, wd, x, d, f, out=out, h_scratch=h)
    x3 = torch.zeros((3, d), dtype=F32)
    refused("workspace: expected torch.uint8", qg.qgemv_q8act, "q4_0", wg, x3, f, d,
            workspace=torch.zeros(qg.q8act_workspace_bytes("q4_0", f, d, 3), dtype=F32))


def test_head_argmax_quantize_dequant_repack_refusals():
    pk, x = packed("q8_0", R, C), torch.zeros(C, dtype=F32)
    refused("token: expected torch.int32", qg.qgemv_argmax, torch.zeros(R, dtype=F32), R,
            token=torch.zeros(1, dtype=torch.int64))
    refused("whole number of rows", qg.qgemv_argmax, torch.zeros(R + 3, dtype=F32), R)
    refused("logits: needs at least", qg.qgemv_head_argmax, "q8_0", pk, x, R, C,
            logits=torch.zeros(R - 1, dtype=F32), token=torch.zeros(1, dtype=I32))
    refused("token: needs at least", qg.qgemv_head_argmax, "q8_0", pk, torch.zeros(2 * C, dtype=F32), R, C,
            logits=torch.zeros(2 * R, dtype=F32), token=torch.zeros(1, dtype=I32))
    refused("workspace: needs at least", qg.qgemv_head_argmax, "q8_0", pk, x, R, C,
            workspace=torch.zeros(256 + 8 * R - 1, dtype=U8), fused=True)
    refused("workspace: expected torch.uint8", qg.qgemv_head_argmax, "q8_0", pk, x, R, C,
            workspace=torch.zeros(256 + 8 * R, dtype=F32), fused=True)
    assert qg.head_argmax_workspace_bytes("q8_0", R, C) == 256 + 8 * R
    refused("blocks: needs at least", qg.qquantize_q8_0, x, C, blocks=torch.zeros(C // 32 * 34 - 1, dtype=U8))
    refused("w_out: needs at least", qg.qdequant, "q8_0", pk, R, C, w_out=torch.zeros(R * C - 1, dtype=F32))
    refused("raw: needs at least", qg.qgemv_repack_q4_0, torch.zeros(R * (C // 32) * 18 - 1, dtype=U8),
            packed("q4_0", R, C), R, C)
    refused("raw: expected torch.uint8", qg.qgemv_repack_q4_k, torch.zeros(R * (C // 256) * 144, dtype=I8),
            packed("q4_k", R, C), R, C)
    refused("row_scale: expected torch.float32", qg.qgemv_repack_i8row, torch.zeros(R * C, dtype=I8),
            torch.zeros(R, dtype=torch.float64), packed("i8row", R, C), R, C)
    refused("q: expected torch.int8", qg.qgemv_repack_i8row, torch.zeros(R * C, dtype=U8),
            torch.zeros(R, dtype=F32), packed("i8row", R, C), R, C)
    refused("packed: needs at least", qg.qgemv_repack_q6_k, torch.zeros(R * (C // 256) * 210, dtype=U8),
            packed("q6_k", R, C)[:-1], R, C)
