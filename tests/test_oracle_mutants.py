"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them."""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import pins

# (name, text in w4a16_oracle.c, replacement)
MUTANTS = [
    ("no_mask_after_shift", "int uval = (int)((word >> (4 * (k % 8))) & 0xFu);",
     "int uval = (int)((word >> (4 * (k % 8))));"),
    ("signed_shift_no_mask", "uint32_t word = (uint32_t)packed[(k / 8) * N + n];\n    int uval = (int)((word >> (4 * (k % 8))) & 0xFu);",
     "int32_t word = packed[(k / 8) * N + n];\n    int uval = (int)(word >> (4 * (k % 8)));"),
    ("unpack_no_mask", "u[k * N + n] = (uint8_t)((word >> (4 * (k % 8))) & 0xFu);",
     "u[k * N + n] = (uint8_t)((word >> (4 * (k % 8))));"),
    ("round_half_away", "float q = nearbyintf(r);", "float q = roundf(r);"),
    ("divide_by_8", "float s = amax / 7.0f;", "float s = amax / 8.0f;"),
    ("offset_7_quantize", "u[k * N + n] = (uint8_t)((int)q + 8);", "u[k * N + n] = (uint8_t)((int)q + 7);"),
    ("offset_7_dequant", "return (double)(uval - 8) *", "return (double)(uval - 7) *"),
    ("reversed_nibble_order", "word |= ((uint32_t)(u[(8 * r + i) * N + n] & 0xF)) << (4 * i);",
     "word |= ((uint32_t)(u[(8 * r + (7 - i)) * N + n] & 0xF)) << (4 * i);"),
    ("scale_from_wrong_column", "(uval - 8) * oracle_f16_to_f64(s16[(k / G) * N + n]);",
     "(uval - 8) * oracle_f16_to_f64(s16[(k / G) * N + (N - 1 - n)]);"),
    ("gemm_dropped_term", "for (int64_t k = 0; k < K; ++k) {\n                double a = oracle_f16_to_f64(A16[m * K + k]);\n                for (int64_t n = n0; n < n1; ++n)\n                    acc[n - n0] += a * exact_weight",
     "for (int64_t k = 1; k < K; ++k) {\n                double a = oracle_f16_to_f64(A16[m * K + k]);\n                for (int64_t n = n0; n < n1; ++n)\n                    acc[n - n0] += a * exact_weight"),
    ("gemm_transposed_A", "double a = oracle_f16_to_f64(A16[m * K + k]);\n                for (int64_t n = n0; n < n1; ++n)\n                    acc[n - n0] += a * exact_weight",
     "double a = oracle_f16_to_f64(A16[k * M + m]);\n                for (int64_t n = n0; n < n1; ++n)\n                    acc[n - n0] += a * exact_weight"),
    ("f16_ties_away", "double n = nearbyint(a / ldexp(1.0, e - 10));", "double n = round(a / ldexp(1.0, e - 10));"),
    ("f16_decode_bias", "v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    ("f16_subnormal_quantum", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -23);"),
    ("swiglu_swapped", "double g = C[m * N + j];\n            double up = C[m * N + I + j];",
     "double up = C[m * N + j];\n            double g = C[m * N + I + j];"),
    ("silu_sign", "g / (1.0 + exp(-g)) * up", "g / (1.0 + exp(g)) * up"),
    ("scale_clamp_dropped_zero_group", "float s = amax / 7.0f;\n            if (s < 1e-8f)\n                s = 1e-8f;",
     "float s = amax / 7.0f;\n            if (s < 1e-8f)\n                s = 1.0f;"),
    ("int8_scale_clamp_dropped_zero_group", "float s = amax / 127.0f;\n            if (s < 1e-8f)\n                s = 1e-8f;",
     "float s = amax / 127.0f;\n            if (s < 1e-8f)\n                s = 1.0f;"),
    ("bf16_ties_away", "double n = nearbyint(a / ldexp(1.0, e - 7));", "double n = round(a / ldexp(1.0, e - 7));"),
    ("bf16_decode_bias", "v = ldexp((double)(128 + f), e - 134);", "v = ldexp((double)(128 + f), e - 133);"),
    ("bf16_truncate", "double n = nearbyint(a / ldexp(1.0, e - 7));", "double n = floor(a / ldexp(1.0, e - 7));"),
    ("bf16_gemm_unrounded_weight", "double w = oracle_bf16_to_f64(\n                        oracle_f64_to_bf16(exact_weight(packed, s16, N, G, k, n)));",
     "double w = exact_weight(packed, s16, N, G, k, n);"),
    ("fold_gain_dropped", "Wf[k * N + n] = (float)((double)gamma[k] * (double)W[k * N + n]);",
     "Wf[k * N + n] = W[k * N + n];"),
    ("fold_gain_wrong_index", "Wf[k * N + n] = (float)((double)gamma[k] * (double)W[k * N + n]);",
     "Wf[k * N + n] = (float)((double)gamma[n % K] * (double)W[k * N + n]);"),
    ("rms_mean_over_k_minus_1", "rho[m] = 1.0 / sqrt(q / (double)K + eps);", "rho[m] = 1.0 / sqrt(q / (double)(K - 1) + eps);"),
    ("rms_eps_dropped", "rho[m] = 1.0 / sqrt(q / (double)K + eps);", "rho[m] = 1.0 / sqrt(q / (double)K);"),
    ("rms_no_sqrt", "rho[m] = 1.0 / sqrt(q / (double)K + eps);", "rho[m] = 1.0 / (q / (double)K + eps);"),
    ("scale_rows_by_column", "out[m * N + n] = rho[m] * C[m * N + n];", "out[m * N + n] = rho[n % M] * C[m * N + n];"),
    ("bf16_gemm_fp16_activations", "double a = oracle_bf16_to_f64(Ab[m * K + k]);\n                for (int64_t n = n0; n < n1; ++n) {",
     "double a = oracle_f16_to_f64(Ab[m * K + k]);\n                for (int64_t n = n0; n < n1; ++n) {"),
    ("gemm_wb_fp16_activations", "double a = oracle_bf16_to_f64(Ab[m * K + k]);\n                for (int64_t n = n0; n < n1; ++n)\n                    acc[n - n0] += a * oracle_bf16_to_f64(Wb",
     "double a = oracle_f16_to_f64(Ab[m * K + k]);\n                for (int64_t n = n0; n < n1; ++n)\n                    acc[n - n0] += a * oracle_bf16_to_f64(Wb"),
    ("zero_point_sign", "z16[i] = oracle_f64_to_f16((8.0 - (double)zp[i]) * oracle_f16_to_f64(s16[i]));",
     "z16[i] = oracle_f64_to_f16(((double)zp[i] - 8.0) * oracle_f16_to_f64(s16[i]));"),
    ("zero_point_offset_7", "z16[i] = oracle_f64_to_f16((8.0 - (double)zp[i]) * oracle_f16_to_f64(s16[i]));",
     "z16[i] = oracle_f64_to_f16((7.0 - (double)zp[i]) * oracle_f16_to_f64(s16[i]));"),
    ("zero_row_bf16_rounded", "z16[i] = oracle_f64_to_f16((8.0 - (double)zp[i]) * oracle_f16_to_f64(s16[i]));",
     "z16[i] = oracle_f64_to_f16(oracle_bf16_to_f64(oracle_f64_to_bf16((8.0 - (double)zp[i]) * oracle_f16_to_f64(s16[i]))));"),
    ("zero_point_two_roundings", "double w = exact_weight_zp(packed, s16, z16, N, G, k, n);",
     "double w = oracle_f16_to_f64(oracle_f64_to_f16(exact_weight(packed, s16, N, G, k, n))) + oracle_f16_to_f64(z16[(k / G) * N + n]);"),
    ("zero_row_wrong_group", "return exact_weight(packed, s16, N, G, k, n) + oracle_f16_to_f64(z16[(k / G) * N + n]);",
     "return exact_weight(packed, s16, N, G, k, n) + oracle_f16_to_f64(z16[(k / 128) * N + n]);"),
    ("zero_row_dropped", "return exact_weight(packed, s16, N, G, k, n) + oracle_f16_to_f64(z16[(k / G) * N + n]);",
     "return exact_weight(packed, s16, N, G, k, n);"),
    ("zero_point_bf16_flag_ignored", "double w = exact_weight_zp(packed, s16, z16, N, G, k, n);\n            W[k * N + n] = bf16 ? oracle_f64_to_bf16(w) : oracle_f64_to_f16(w);",
     "double w = exact_weight_zp(packed, s16, z16, N, G, k, n);\n            W[k * N + n] = oracle_f64_to_f16(w);"),
    ("int8_bf16_flag_ignored", "double w = exact_weight8(packed, s16, N, G, k, n);\n            W[k * N + n] = bf16 ? oracle_f64_to_bf16(w) : oracle_f64_to_f16(w);",
     "double w = exact_weight8(packed, s16, N, G, k, n);\n            W[k * N + n] = oracle_f64_to_f16(w);"),
    ("int8_divide_by_128", "float s = amax / 127.0f;", "float s = amax / 128.0f;"),
    ("int8_offset_127", "u[k * N + n] = (uint8_t)((int)q + 128);", "u[k * N + n] = (uint8_t)((int)q + 127);"),
    ("int8_clamp_upper_126", "if (q > 127.0f)\n                    q = 127.0f;", "if (q > 126.0f)\n                    q = 126.0f;"),
    ("int8_round_half_away", "float q = nearbyintf(W[k * N + n] / s); /* ties to even */",
     "float q = roundf(W[k * N + n] / s); /* ties to even */"),
    ("int8_pack_reversed", "word |= (uint32_t)u[(4 * r + i) * N + n] << (8 * i);",
     "word |= (uint32_t)u[(4 * r + (3 - i)) * N + n] << (8 * i);"),
    ("int8_unpack_nibble_shift", "u[k * N + n] = (uint8_t)((word >> (8 * (k % 4))) & 0xFFu);",
     "u[k * N + n] = (uint8_t)((word >> (4 * (k % 4))) & 0xFFu);"),
    ("int8_dequant_bias_127", "return (double)(uval - 128) * oracle_f16_to_f64(s16[(k / G) * N + n]);",
     "return (double)(uval - 127) * oracle_f16_to_f64(s16[(k / G) * N + n]);"),
    ("int8_weight_scale_group_128", "return (double)(uval - 128) * oracle_f16_to_f64(s16[(k / G) * N + n]);",
     "return (double)(uval - 128) * oracle_f16_to_f64(s16[(k / 128) * N + n]);"),
    ("int8_gemm_bf16_unrounded", "if (bf16)\n                        w = oracle_bf16_to_f64(oracle_f64_to_bf16(w));",
     "if (0)\n                        w = oracle_bf16_to_f64(oracle_f64_to_bf16(w));"),
    ("int8_gemm_dropped_term", "for (int64_t k = 0; k < K; ++k) {\n                double a = bf16 ? oracle_bf16_to_f64",
     "for (int64_t k = 1; k < K; ++k) {\n                double a = bf16 ? oracle_bf16_to_f64"),
    ("gemm_wb_fp16_weights", "acc[n - n0] += a * oracle_bf16_to_f64(Wb[k * N + n]);",
     "acc[n - n0] += a * oracle_f16_to_f64(Wb[k * N + n]);"),
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def _run_checks(o):
    failed = []
    for check in pins.FAST_CHECKS:
        try:
            check(o)
        except (AssertionError, ValueError) as e:  # noqa: PERF203
            failed.append(check.__name__)
    return failed


def test_mutant_list_applies():
    src = open(oracle.SOURCE).read()
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(workdir, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1
    path = os.path.join(workdir, name + ".c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(path, os.path.join(workdir, "lib_%s.so" % name))
    failed = _run_checks(oracle.Oracle(lib))
    assert failed, "no pin caught mutant %s" % name
