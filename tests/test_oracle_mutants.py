"""The pins have teeth: each plausible mistake, planted in a temporary copy of
the oracle's C source (never in the committed file), makes at least one pin
fail. Runs on the CPU only."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "qmv_oracle.c")

MUTANTS = {
    "q4_0_nibble_halves_swapped": ("int q = (e < 16) ? (qs[e] & 0x0f) : (qs[e - 16] >> 4)",
                                   "int q = (e < 16) ? (qs[e] >> 4) : (qs[e - 16] & 0x0f)"),
    "q4_0_offset_7": ("d * (float)(q - 8)", "d * (float)(q - 7)"),
    "q4_k_scale_high_bits_wrong_byte": ("*scale = (sc[s + 4] & 0x0f) | ((sc[s - 4] >> 6) << 4);",
                                        "*scale = (sc[s + 4] & 0x0f) | ((sc[s] >> 6) << 4);"),
    "q4_k_min_high_bits_wrong_byte": ("*min = (sc[s + 4] >> 4) | ((sc[s] >> 6) << 4);",
                                      "*min = (sc[s + 4] >> 4) | ((sc[s - 4] >> 6) << 4);"),
    "q4_k_min_sign": ("return a - b;", "return a + b;"),
    "q4_k_nibble_order": ("(qs[32 * c + l] >> (4 * h))", "(qs[32 * c + l] >> (4 * (1 - h)))"),
    "q4_k_low_slots_swapped": ("*scale = sc[s] & 63;\n        *min = sc[s + 4] & 63;",
                               "*scale = sc[s + 4] & 63;\n        *min = sc[s] & 63;"),
    "q6_k_qh_shift": (">> (2 * g)) & 3", ">> (2 * (g ^ 1))) & 3"),
    "q6_k_scale_index": ("scales[8 * h + 2 * g + l / 16]", "scales[8 * h + g + l / 16]"),
    "q6_k_ql_half": ("ql[64 * h + 32 * (g % 2) + l]", "ql[64 * h + 32 * (g / 2) + l]"),
    "q6_k_offset_31": ("(float)(q - 32)", "(float)(q - 31)"),
    "q6_k_unsigned_scales": ("const int8_t *scales = (const int8_t *)(blk + 192);",
                             "const uint8_t *scales = (const uint8_t *)(blk + 192);"),
    "f16_subnormal_scale": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "f16_exponent_bias": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    "bf16_wrong_half": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "gemv_drops_first_term": ("for (int64_t i = 0; i < k; i++) {\n                double p",
                              "for (int64_t i = 1; i < k; i++) {\n                double p"),
    "gemv_x_index_transposed": ("(double)x[t * k + i] * (double)w[i]",
                                "(double)x[i * m + t] * (double)w[i]"),
    "gemv_bound_signed": ("mag += fabs(p);\n            }\n            y[t * nrows + r]",
                          "mag += p;\n            }\n            y[t * nrows + r]"),
    "gemv_t_bound_signed": ("mag += fabs(p);\n            }\n            dx[t * ncols + c]",
                            "mag += p;\n            }\n            dx[t * ncols + c]"),
    "q6_k_d_offset": ("rd_u16(blk + 208)", "rd_u16(blk + 206)"),
    "q8_0_unsigned_codes": ("int q = (int)(int8_t)blk[2 + e];", "int q = (int)blk[2 + e];"),
    "q8_0_code_offset": ("int q = (int)(int8_t)blk[2 + e];", "int q = (int)(int8_t)blk[1 + e];"),
    "q5_0_fifth_bit_low_half_only": ("int hi = (int)((qh >> e) & 1u);",
                                     "int hi = (int)((qh >> (e % 16)) & 1u);"),
    "q5_0_offset_15": ("return d * (float)(q - 16);", "return d * (float)(q - 15);"),
    "q5_0_nibble_halves_swapped": ("int lo = (e < 16) ? (qs[e] & 0x0f) : (qs[e - 16] >> 4);",
                                   "int lo = (e < 16) ? (qs[e] >> 4) : (qs[e - 16] & 0x0f);"),
    "q5_0_qh_big_endian": ("uint32_t qh = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8)",
                           "uint32_t qh = (uint32_t)blk[5] | ((uint32_t)blk[3] << 8)"),
    "q5_0_codes_at_byte_2": ("const uint8_t *qs = blk + 6;", "const uint8_t *qs = blk + 2;"),
    "gemv_t_dy_index_transposed": ("(double)dy[t * n + j] * (double)oracle_elem",
                                   "(double)dy[j * m + t] * (double)oracle_elem"),
    "gemv_t_range_inclusive": ("for (int64_t j = j0; j < j1; j++) {\n                double p = (double)dy",
                               "for (int64_t j = j0; j <= j1 && j < n; j++) {\n                double p = (double)dy"),
    "gemv_t_skips_first_row": ("for (int64_t j = j0; j < j1; j++) {\n                double p = (double)dy",
                               "for (int64_t j = j0 + 1; j < j1; j++) {\n                double p = (double)dy"),
    "gemv_t_row_as_column": ("oracle_elem(fmt, W + j * rb, i)", "oracle_elem(fmt, W + i * rb, j % k)"),
    "affine_codes_high_first": ("uint32_t q = (w >> (bits * (int)(i % per))) & mask;",
                                "uint32_t q = (w >> (bits * (per - 1 - (int)(i % per)))) & mask;"),
    "affine_group_of_32": ("float sc = oracle_bf16_to_f32(scales[i / 64]);",
                           "float sc = oracle_bf16_to_f32(scales[i / 32 % (64 / 32)]);"),
    "affine_bias_sign": ("return (float)q * sc + bi;", "return (float)q * sc - bi;"),
    "affine_scale_bias_swapped": ("float sc = oracle_bf16_to_f32(scales[i / 64]);\n    float bi = oracle_bf16_to_f32(biases[i / 64]);",
                                  "float sc = oracle_bf16_to_f32(biases[i / 64]);\n    float bi = oracle_bf16_to_f32(scales[i / 64]);"),
    "affine_nibble_mask_wide": ("uint32_t mask = (bits == 8) ? 0xffu : 0x0fu;",
                                "uint32_t mask = (bits == 8) ? 0xffu : 0x1fu;"),
}


@pytest.fixture(scope="module")
def src_text():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, src_text, tmp_path):
    old, new = MUTANTS[name]
    assert src_text.count(old) == 1, "mutation site for %s not unique/found" % name
    csrc = tmp_path / "mutant.c"
    csrc.write_text(src_text.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-o", str(so), str(csrc), "-lm"], check=True)
    lib = oracle.load_library(str(so))
    prev = oracle.use_library(lib)
    caught = []
    try:
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                caught.append(pin.__name__)
    finally:
        oracle.use_library(prev)
    assert caught, "no pin caught mutant %s" % name
