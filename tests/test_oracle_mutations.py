"""Plausible mistakes planted in copies of the CPU oracle must each fail a pin.

Each mutant is the oracle's C source with one textual change, compiled into a
temporary directory with the oracle's own flags.  The mistakes cover every
step: nibble order, the block range, rounding, the scale divisor, the code
formula, the zero point's sign, the dequantization formula and its block
index, the matmul's bias, indexing and accumulation precision, the bound, the
head's scale and rounding, and the fused epilogues (GELU's constants, SiLU's
sign, the SwiGLU pairing, the order of activation and residual) and the
group-64 affine variant (range, offset, rounding, the single-rounding
dequantization, its K-major copy).  A mutant
that passes every pin would mean the pins cannot tell that mistake from the
correct oracle.
"""
import os
import shutil

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTATIONS = {
    "g64_range_includes_zero": (
        "            float lo = w[0], hi = w[0];",
        "            float lo = fminf(w[0], 0.0f), hi = fmaxf(w[0], 0.0f);"),
    "g64_offset_is_max": (
        "            mins[g * N + n] = lo;",
        "            mins[g * N + n] = hi;"),
    "g64_truncates": (
        "qv = clamp_int(rintf(d / sc), 0, 15);",
        "qv = clamp_int(truncf(d / sc), 0, 15);"),
    "g64_dequant_two_roundings": (
        "W_hat[k * N + n] = fmaf((float)q[k * N + n], scales[grp], mins[grp]);",
        "W_hat[k * N + n] = (float)q[k * N + n] * scales[grp] + mins[grp];"),
    "g64_prepack_mins_are_scales": (
        "            Pm[n * ng + g] = mins[g * N + n];",
        "            Pm[n * ng + g] = scales[g * N + n];"),
    "gelu_coefficient_typo": (
        "return 0.5 * v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));",
        "return 0.5 * v * (1.0 + tanh(c * (v + 0.44715 * v * v * v)));"),
    "gelu_missing_half": (
        "return 0.5 * v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));",
        "return v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));"),
    "silu_sign": (
        "return v / (1.0 + exp(-v));",
        "return v / (1.0 + exp(v));"),
    "swiglu_pair_swapped": (
        "const double g = t[2 * i], u = t[2 * i + 1], sg = orc_silu(g);",
        "const double g = t[2 * i + 1], u = t[2 * i], sg = orc_silu(g);"),
    "gelu_bound_slope_loose": (
        "b = 1.13 * tb[i] + ldexp(fabs(t[i]) + fabs(o), -20);",
        "b = 11.3 * tb[i] + ldexp(fabs(t[i]) + fabs(o), -20);"),
    "gelu_bound_slope_too_small": (
        "b = 1.13 * tb[i] + ldexp(fabs(t[i]) + fabs(o), -20);",
        "b = 0.9 * tb[i] + ldexp(fabs(t[i]) + fabs(o), -20);"),
    "swiglu_bound_drops_gate_error": (
        "b = 1.1 * fabs(u) * tb[2 * i] + fabs(sg) * tb[2 * i + 1] +",
        "b = fabs(sg) * tb[2 * i + 1] +"),
    "swiglu_bound_slope_loose": (
        "b = 1.1 * fabs(u) * tb[2 * i] + fabs(sg) * tb[2 * i + 1] +",
        "b = 11.0 * fabs(u) * tb[2 * i] + fabs(sg) * tb[2 * i + 1] +"),
    "epilogue_residual_before_act": (
        "                o = orc_gelu(t[i]);",
        "                o = orc_gelu(t[i] + (residual ? (double)residual[m * nout + i] : 0.0));"),

    "f16_truncates": (
        "double units = rint(a / quantum); /* in [0, 2048] */",
        "double units = floor(a / quantum); /* in [0, 2048] */"),
    "f16_flushes_subnormals": (
        "if (v < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)units); /* subnormal */",
        "if (v < ldexp(1.0, -14)) return sign; /* subnormal */"),
    "f16_overflow_at_max": (
        "if (a >= 65520.0) return (uint16_t)(sign | 0x7C00);",
        "if (a > 65504.0) return (uint16_t)(sign | 0x7C00);"),
    "f16_codes_against_fp32_scale": (
        "s = orc_f16_to_f32(h); /* the stored value */",
        "s = h ? s : 0.0f; /* the stored value */"),
    "f16_decode_bias_14": (
        "else v = ldexp(1.0 + fr / 1024.0, ex - 15);",
        "else v = ldexp(1.0 + fr / 1024.0, ex - 14);"),
    "pack_high_nibble_first": (
        "out[i] = (uint8_t)((v[2 * i] & 15) | ((v[2 * i + 1] & 15) << 4));",
        "out[i] = (uint8_t)((v[2 * i + 1] & 15) | ((v[2 * i] & 15) << 4));"),
    "unpack_high_nibble_first": (
        "v[2 * i] = (uint8_t)(in[i] & 15);\n        v[2 * i + 1] = (uint8_t)(in[i] >> 4);",
        "v[2 * i + 1] = (uint8_t)(in[i] & 15);\n        v[2 * i] = (uint8_t)(in[i] >> 4);"),
    "range_without_zero": (
        "float lo = 0.0f, hi = 0.0f;",
        "float lo = w[0], hi = w[0];"),
    "round_half_away": (
        "float t = rintf(w[r * stride] / s);",
        "float t = roundf(w[r * stride] / s);"),
    "round_down": (
        "float t = rintf(w[r * stride] / s);",
        "float t = floorf(w[r * stride] / s);"),
    "scale_over_16": (
        "float s = range / 15.0f;",
        "float s = range / 16.0f;"),
    "code_from_range_start": (
        "q_out[r] = (uint8_t)clamp_int(t + (float)z, 0, 15);",
        "q_out[r] = (uint8_t)clamp_int(rintf((w[r * stride] - lo) / s), 0, 15);"),
    "zero_point_sign": (
        "float zr = rintf(-lo / s);",
        "float zr = rintf(lo / s);"),
    "dequant_drops_zero_point": (
        "int diff = (int)q[k * N + n] - (int)z[blk];",
        "int diff = (int)q[k * N + n];"),
    "dequant_scales_transposed": (
        "int64_t blk = (k / BLOCK) * N + n;",
        "int64_t blk = n * (K / BLOCK) + (k / BLOCK);"),
    "quantize_scale_stored_transposed": (
        "st = quantize_block(W + (b * BLOCK) * N + n, N, &scales[b * N + n], NULL,",
        "st = quantize_block(W + (b * BLOCK) * N + n, N, &scales[n * nb + b], NULL,"),
    "matmul_drops_bias": (
        "acc += (double)bias[n];",
        "acc += 0.0;"),
    "matmul_weight_transposed": (
        "double p = (double)xr[k] * (double)W[k * N + n];",
        "double p = (double)xr[k] * (double)W[n * K + k];"),
    "matmul_fp32_accumulation": (
        "double acc = 0.0, mag = 0.0;",
        "float acc = 0.0f; double mag = 0.0;"),
    "bound_uses_abs_of_sum": (
        "tb[n] = 1e-5 * mag + 1e-6;",
        "tb[n] = 1e-5 * fabs(acc) + 1e-6;"),
    "head_scale_over_128": (
        "float s = amax / 127.0f;",
        "float s = amax / 128.0f;"),
    "head_truncates": (
        "if (s != 0.0f) qv = clamp_int(rintf(E[k * N + n] / s), -127, 127);",
        "if (s != 0.0f) qv = clamp_int(truncf(E[k * N + n] / s), -127, 127);"),
    "prepack_scales_not_transposed": (
        "            Ps[n * nb + b] = scales[b * N + n];",
        "            Ps[b * N + n] = scales[b * N + n];"),
    "prepack_codes_not_transposed": (
        "        for (int64_t n = 0; n < N; ++n) qt[n * K + k] = q[k * N + n];",
        "        for (int64_t n = 0; n < N; ++n) qt[k * N + n] = q[k * N + n];"),
    "embed_wrong_scale": (
        "out[t * K + k] = (float)((double)Q[k * ldq + tok] * (double)hs[tok]);",
        "out[t * K + k] = (float)((double)Q[k * ldq + tok] * (double)hs[k]);"),
}


@pytest.fixture(scope="module")
def source():
    with open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTATIONS[name]
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    d = tmp_path / name
    d.mkdir()
    shutil.copy(os.path.join(os.path.dirname(oracle.__file__), "oracle.h"), d / "oracle.h")
    (d / "oracle.c").write_text(source.replace(old, new))
    so = oracle.build(str(d / "oracle.c"), str(d / "liboracle_mutant.so"))
    orc = oracle.Oracle(oracle.load_library(so))
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, oracle.OracleError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
