"""The oracle's pins must reject plausible mistakes.

Each case plants one mistake in a copy of oracle/sgmv_oracle.c (on the CPU,
in a temporary directory), builds it with gcc, routes the oracle through it
and runs the pin tests of test_oracle.py; at least one pin must fail.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sgmv_oracle.c")

MUTANTS = {
    "A_read_transposed": ("acc += decode(dtype, x_row[h]) * decode(dtype, a[(int64_t)h * rank + j]);",
                          "acc += decode(dtype, x_row[h]) * decode(dtype, a[(int64_t)j * h_in + h]);"),
    "B_read_transposed": ("acc += v[j] * decode(dtype, b[(int64_t)j * h_out + c]);",
                          "acc += v[j] * decode(dtype, b[(int64_t)c * rank + j]);"),
    "base_output_dropped": ("y[c] = decode(dtype, y0_row[c]) + scale * acc;", "y[c] = scale * acc;"),
    "term_sign_flipped": ("y[c] = decode(dtype, y0_row[c]) + scale * acc;",
                          "y[c] = decode(dtype, y0_row[c]) - scale * acc;"),
    "scale_ignored": ("y[c] = decode(dtype, y0_row[c]) + scale * acc;",
                      "y[c] = decode(dtype, y0_row[c]) + acc;"),
    "scale_applied_to_base": ("y[c] = decode(dtype, y0_row[c]) + scale * acc;",
                              "y[c] = scale * (decode(dtype, y0_row[c]) + acc);"),
    "rank_table_short_by_one_vector": ("const int32_t rk = ranks ? ranks[k] : rank;",
                                       "const int32_t rk = ranks ? (ranks[k] > 8 ? ranks[k] - 8 : 0) : rank;"),
    "segment_index_as_lora": ("const int32_t k = lora_idx[s];\n", "const int32_t k = s % num_loras;\n"),
    "base_segment_index_as_lora": ("const int32_t k = lora_idx[s];  /* LoRA",
                                   "const int32_t k = s % num_loras;  /* LoRA"),
    "last_row_of_segment_dropped": ("for (int32_t i = lo; i < hi; ++i) seg_of_row[i] = s;",
                                    "for (int32_t i = lo; i + 1 < hi; ++i) seg_of_row[i] = s;"),
    "first_input_column_dropped": ("for (int32_t h = 0; h < h_in; ++h)\n      acc +=",
                                   "for (int32_t h = 1; h < h_in; ++h)\n      acc +="),
    "base_weight_transposed": ("y[c] += xh * decode(dtype, w_row[c]);",
                               "y[c] += xh * decode(dtype, W[(int64_t)c * h_in + h]);"),
    "base_term_dropped": ("y[c] += xh * decode(dtype, w_row[c]);", "y[c] += 0.0 * xh * decode(dtype, w_row[c]);"),
    "base_first_input_row_dropped": ("for (int32_t h = 0; h < h_in; ++h) {  /* base",
                                     "for (int32_t h = 1; h < h_in; ++h) {  /* base"),
    "base_lora_term_subtracted": ("      y[c] += acc;", "      y[c] -= acc;"),
    "base_last_rank_dropped": ("for (int32_t j = 0; j < rank; ++j)  /* LoRA term",
                               "for (int32_t j = 0; j + 1 < rank; ++j)  /* LoRA term"),
    "base_lora_from_first_row": ("row_shrink(dtype, h_in, rank, x_row, A[k], v);",
                                 "row_shrink(dtype, h_in, rank, X, A[k], v);"),
    "last_rank_dropped": ("for (int32_t j = 0; j < rank; ++j) acc += v[j]",
                          "for (int32_t j = 0; j + 1 < rank; ++j) acc += v[j]"),
    "f16_subnormal_scale": ("mag = ldexp((double)frac, -24);", "mag = ldexp((double)frac, -25);"),
    "f16_exponent_bias": ("mag = ldexp((double)(1024 + frac), expo - 25);",
                          "mag = ldexp((double)(1024 + frac), expo - 24);"),
    "bf16_wrong_half": ("const uint32_t word = (uint32_t)bits << 16;",
                        "const uint32_t word = (uint32_t)bits << 15;"),
    "uncovered_rows_zeroed": ("for (int32_t c = 0; c < h_out; ++c) y[c] = decode(dtype, y0[c]);\n      continue;\n    }\n    double v[4096];",
                              "for (int32_t c = 0; c < h_out; ++c) y[c] = 0.0;\n      continue;\n    }\n    double v[4096];"),
}

PINS = [
    pins.test_decode_every_f16_pattern,
    pins.test_decode_every_bf16_pattern,
    pins.test_decode_known_values,
    pins.test_golden_closed_form_example,
    pins.test_merge_identity_of_lora_paragraph,
    lambda: pins.test_identical_popularity_is_one_dense_product("f16"),
    lambda: pins.test_identical_popularity_is_one_dense_product("bf16"),
    lambda: pins.test_tiny_workload_brute_force("f16"),
    lambda: pins.test_tiny_workload_brute_force("bf16"),
    pins.test_uncovered_rows_keep_base_output,
    pins.test_segments_equal_per_row_definition,
    lambda: pins.test_rank_table_equals_zero_padding("f16"),
    pins.test_rank_zero_lora_adds_nothing,
    pins.test_scale_multiplies_the_term_only,
    lambda: pins.test_base_apply_with_zero_weight_is_the_lora_term("f16"),
    lambda: pins.test_base_apply_without_segments_is_a_matmul("bf16"),
    pins.test_base_apply_identity_weight_adds_the_input,
    pins.test_base_apply_uncovered_rows_get_the_base_term_only,
    lambda: pins.test_base_apply_brute_force("f16"),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", "-o", str(so), str(path), "-lm"], check=True)
    failed = []
    with oracle.using_library(str(so)):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                failed.append(getattr(pin, "__name__", "lambda"))
    assert failed, f"no pin caught the planted mistake {name}"
