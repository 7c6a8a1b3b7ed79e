"""The oracle against its pins, and the pins against planted mistakes in the oracle."""
import json
import os
import subprocess
import sys
from pathlib import Path

import pytest

import oracle
import oracle_pins

ROOT = Path(__file__).resolve().parents[1]


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, orc):
    pin(orc)


# Plausible mistakes, each planted as a text edit of the oracle's C source.  Every one
# must make at least one pin fail; a mutant that passes all pins shows a hole in them.
MUTANTS = {
    "sign_mapping_swapped": ("return bit ? s : -s;", "return bit ? -s : s;"),
    "group_of_64": ("scales[n * (K / 128) + k / 128]);\n    return bit",
                    "scales[n * (K / 128) + (k / 64) % (K / 128)]);\n    return bit"),
    "scale_row_stride": ("scales[n * (K / 128) + k / 128]);\n    return bit",
                         "scales[(n * (K / 128) + k / 128) % (K / 128)]);\n    return bit"),
    "bit_order_reversed": ("(word >> (k % 32)) & 1u;", "(word >> (31 - k % 32)) & 1u;"),
    "word_index_off": ("wbits[n * (K / 32) + k / 32];", "wbits[n * (K / 32) + (k / 32) % 2];"),
    "last_term_dropped": ("for (int64_t k = 0; k < K; ++k) {\n                const double p",
                          "for (int64_t k = 0; k < K - 1; ++k) {\n                const double p"),
    "abs_sum_signed": ("mag += fabs(p);", "mag += p;"),
    "x_transposed": ("bo_f16_to_f64(x[m * K + k])", "bo_f16_to_f64(x[(k * M + m) % (M * K)])"),
    "ternary_codes_swapped": ("case 1: *t = 1; return 0;\n    case 3: *t = -1;",
                              "case 1: *t = -1; return 0;\n    case 3: *t = 1;"),
    "ternary_field_order": ("(word >> (2 * (k % 16))) & 3u;", "(word >> (30 - 2 * (k % 16))) & 3u;"),
    "ternary_reserved_as_zero": ("default: return BO_ERR_CODE;", "default: *t = 0; return 0;"),
    "affine_bias_dropped": ("* q + bo_f16_to_f64(biases[g]);", "* q;"),
    "affine_scale_bias_swapped": ("return bo_f16_to_f64(scales[g]) * q + bo_f16_to_f64(biases[g]);",
                                  "return bo_f16_to_f64(biases[g]) * q + bo_f16_to_f64(scales[g]);"),
    "affine_bit_inverted": ("const double q = (double)((word >> (k % 32)) & 1u);",
                            "const double q = (double)(((~word) >> (k % 32)) & 1u);"),
    "affine_group_of_64": ("const int64_t g = n * (K / 128) + k / 128;",
                           "const int64_t g = n * (K / 128) + (k / 64) % (K / 128);"),
    "t5_digit_order_reversed": ("for (int64_t j = 0; j < i; ++j) place *= 3;",
                                "for (int64_t j = 0; j < 4 - i; ++j) place *= 3;"),
    "t5_five_consecutive_k": ("const int64_t b = k / 160, i = (k % 160) / 32, c = k % 32;",
                              "const int64_t b = k / 160, i = (k % 160) % 5, c = (k % 160) / 5;"),
    "t5_digit_two_as_plus": ("    case 1: *t = 1; return 0;\n    default: *t = -1; return 0;",
                             "    case 1: *t = -1; return 0;\n    default: *t = 1; return 0;"),
    "t5_superblock_stride": ("codes[n * row_bytes + 32 * b + c]", "codes[n * row_bytes + 30 * b + c]"),
    "t5_row_bytes_floor": ("32 * ((K + 159) / 160)", "32 * (K / 160)"),
    "t5_reserved_accepted": ("if (v >= 243) return BO_ERR_CODE;", "if (v > 255) return BO_ERR_CODE;"),
    "f16_bias_off_by_one": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    "f16_subnormal_wrong": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "f16_implicit_bit_dropped": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)f, e - 25)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = (ROOT / "oracle" / "bonsai_oracle.c").read_text()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = oracle.build(mutated, tmp_path / "libmutant.so")
    env = dict(os.environ, PYTHONPATH=f"{ROOT}:{ROOT / 'tests'}")
    out = subprocess.run([sys.executable, str(ROOT / "tests" / "oracle_pins.py"), str(lib)],
                         capture_output=True, text=True, env=env, timeout=300)
    if out.returncode != 0:
        return  # the mutant crashed the pin run: caught
    failed = json.loads(out.stdout.strip().splitlines()[-1])
    assert failed, f"no pin catches the planted mistake {name}"
