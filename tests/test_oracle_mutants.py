"""Plant plausible mistakes in a copy of the oracle and check the pins catch each.

Every mutant is a one-spot edit of oracle.c (a dropped term, a wrong sign, a
wrong index or shift, a transposed output, the other common nibble order),
compiled on the CPU into a temporary library; the oracle pin suite then runs in
a child process against it and must fail.  Nothing here touches a GPU.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_decode.py", "tests/test_oracle_gemv.py", "tests/test_oracle_swiglu.py",
             "tests/test_oracle_norm.py", "tests/test_oracle_argmax.py", "tests/test_oracle_q8act.py"]

MUTANTS = {
    "f16_exponent_bias": ("ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    "f16_subnormal_scale": ("ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    "q8_0_unsigned_codes": ("int q = (int8_t)blk[2 + l];", "int q = blk[2 + l];"),
    "q4_0_interleaved_nibbles": (
        "out[b * 32 + l] = (double)(lo - 8) * d;\n                out[b * 32 + 16 + l] = (double)(hi - 8) * d;",
        "out[b * 32 + 2 * l] = (double)(lo - 8) * d;\n                out[b * 32 + 2 * l + 1] = (double)(hi - 8) * d;"),
    "q4_0_dropped_offset": ("out[b * 32 + l] = (double)(lo - 8) * d;", "out[b * 32 + l] = (double)(lo) * d;"),
    "q4_0_offset_7": ("out[b * 32 + 16 + l] = (double)(hi - 8) * d;", "out[b * 32 + 16 + l] = (double)(hi - 7) * d;"),
    "q4_k_min_added": ("* (double)q - dmin * (double)m", "* (double)q + dmin * (double)m"),
    "q4_k_min_dropped": ("* (double)q - dmin * (double)m", "* (double)q"),
    "q4_k_scale_high_bits_shift": ("((q[j - 4] >> 6) << 4)", "((q[j - 4] >> 4) << 4)"),
    "q4_k_min_high_bits_from_wrong_byte": ("((q[j] >> 6) << 4)", "((q[j - 4] >> 6) << 4)"),
    "q4_k_nibble_parity": ("(s % 2 == 0) ? (chunk[l] & 0x0F)", "(s % 2 == 1) ? (chunk[l] & 0x0F)"),
    "q4_k_chunk_stride": ("qs + 32 * (s / 2)", "qs + 16 * s"),
    "q6_k_offset_31": ("(double)(q - 32)", "(double)(q - 31)"),
    "q6_k_scale_per_32": ("(double)scales[c / 16]", "(double)scales[c / 32]"),
    "q6_k_unsigned_scales": ("const int8_t *scales = (const int8_t *)(blk + 192);",
                             "const uint8_t *scales = (const uint8_t *)(blk + 192);"),
    "q6_k_qh_shift": ("(qh[32 * half + l] >> (2 * j)) & 3", "(qh[32 * half + l] >> j) & 3"),
    "q6_k_ql_half_stride": ("ql[64 * half + 32 * (j % 2) + l]", "ql[32 * half + 32 * (j % 2) + l]"),
    "q6_k_nibble_by_parity": ("(j < 2) ? (lo_byte & 0x0F)", "(j % 2 == 0) ? (lo_byte & 0x0F)"),
    "q6_k_high_bits_low": ("int q = lo | (hi << 4);", "int q = (lo << 2) | hi;"),
    "q6_k_d_first": ("rd_u16(blk + 208)", "rd_u16(blk)"),
    "f16_round_down": ("const double r = nearbyint(a / spacing);", "const double r = floor(a / spacing);"),
    "f16_spacing": ("const double spacing = ldexp(1.0, ue - 10);", "const double spacing = ldexp(1.0, ue - 11);"),
    "q8act_scale_128": ("const float d = amax / 127.0f;", "const float d = amax / 128.0f;"),
    "q8act_truncated_codes": ("(int8_t)roundf(xb[l] * id)", "(int8_t)(xb[l] * id)"),
    "q8act_ties_to_even": ("(int8_t)roundf(xb[l] * id)", "(int8_t)rintf(xb[l] * id)"),
    "q8act_signed_max": ("const float a = fabsf(xb[l]);", "const float a = xb[l];"),
    "q8act_block_scale_index": ("oracle_f16_to_f64(d_bits[j / 32])", "oracle_f16_to_f64(d_bits[j / 64])"),
    "i8row_first_row_scale": ("double s = (double)row_scale[r];", "double s = (double)row_scale[0];"),
    "gemv_output_transposed": ("y[t * nr + (o - row_begin)] = acc;", "y[(o - row_begin) * n_tok + t] = acc;"),
    "gemv_dropped_x": ("double p = row[j] * (double)xt[j];", "double p = row[j];"),
    "gemv_signed_magnitude": ("mag += fabs(p);\n            }\n            y[t * nr", "mag += p;\n            }\n            y[t * nr"),
    "silu_sign": ("return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    "swiglu_gate_up_swapped": ("h[i] = oracle_silu(g[i]) * u[i];\n    return", "h[i] = oracle_silu(u[i]) * g[i];\n    return"),
    "rmsnorm_eps_outside_root": ("1.0 / sqrt(ss / (double)n + eps)", "1.0 / (sqrt(ss / (double)n) + eps)"),
    "rmsnorm_sum_not_mean": ("sqrt(ss / (double)n + eps)", "sqrt(ss + eps)"),
    "rmsnorm_gain_dropped": ("* sc * (double)gamma[j]", "* sc"),
    "rmsnorm_scale_dropped": ("(double)xt[j] * sc * (double)gamma[j]", "(double)xt[j] * (double)gamma[j]"),
    "block_residual_dropped": ("out[i] = (double)x[i] + d[i];", "out[i] = d[i];"),
    "argmax_last_on_ties": ("if (v[i] > v[best])", "if (v[i] >= v[best])"),
    "argmax_skips_first": ("int64_t best = 0;\n    for (int64_t i = 1;", "int64_t best = 1;\n    for (int64_t i = 1;"),
    "block_gate_up_swapped": ("h[i] = oracle_silu(g[i]) * u[i];\n    st =", "h[i] = oracle_silu(u[i]) * g[i];\n    st ="),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/not found"
    mpath = tmp_path / "oracle_mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = obuild.build(out=str(tmp_path / "liboracle_mutant.so"), src=str(mpath), werror=False)
    env = dict(os.environ, ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
