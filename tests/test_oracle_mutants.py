"""Planted mistakes in a copy of the oracle (on the CPU): every plausible
mistake listed here must make at least one pin fail. This shows the pins
would catch that mistake in the oracle itself."""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "qg_oracle.c")

# (name, exact text in qg_oracle.c, replacement)
MUTANTS = [
    ("u4_nibbles_swapped", "(k % 2 == 0) ? (byte & 0x0f) : (byte >> 4)",
     "(k % 2 == 1) ? (byte & 0x0f) : (byte >> 4)"),
    ("b1_msb_first", "(byte >> (k % 8)) & 1", "(byte >> (7 - k % 8)) & 1"),
    ("b1_sign_flipped", "return bit ? sc : -sc;", "return bit ? -sc : sc;"),
    ("u4_bias_dropped", "* (double)q + oracle_bf16_value(b[g])", "* (double)q"),
    ("u4_one_scale_per_row", "int64_t g = m * (K / 64) + k / 64;", "int64_t g = m * (K / 64);"),
    ("u4_scales_transposed", "int64_t g = m * (K / 64) + k / 64;",
     "int64_t g = (k / 64) * A->M + m;"),
    ("i8_read_unsigned", "const int8_t *q = (const int8_t *)A->codes;",
     "const uint8_t *q = (const uint8_t *)A->codes;"),
    ("i8_scale_dropped", "return (double)s[m] * (double)q[m * K + k];",
     "(void)s; return (double)q[m * K + k];"),
    ("fp16_subnormal_as_normal", "v = ldexp((double)f, -24);", "v = ldexp((double)(1024 + f), -25);"),
    ("fp16_exponent_bias", "v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    ("bf16_shift", "uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    ("x_first_row_only", "(double)x[n * A->K + k]", "(double)x[k]"),
    ("absdot_signed", "mag += fabs(p);", "mag += p;"),
    ("argmax_ties_highest", "if (row[m] > row[best])", "if (row[m] >= row[best])"),
    ("b1_group_scale_per_row", "oracle_fp16_value(s[m * (K / 128) + k / 128])",
     "oracle_fp16_value(s[m * (K / 128)])"),
    ("f16_ties_away", "if (rem > half || (rem == half && (r & 1)))", "if (rem >= half)"),
    ("f16_ties_down", "if (rem > half || (rem == half && (r & 1)))", "if (rem > half)"),
    ("f16_no_subnormals", "int qe = L - 10 > -24 ? L - 10 : -24;", "int qe = L - 10;"),
    ("f16_zero_loses_sign", "        return sign;\n", "        return 0;\n"),
    ("f16_no_overflow", "if (e16 >= 31)", "if (e16 >= 32)"),
    ("embed_no_f16_round_trip", "v = (float)oracle_fp16_value(oracle_f32_to_f16(a));", "v = a;"),
    ("embed_bias_dropped", "const float a = prod + b;", "const float a = prod + 0.0f * b;"),
    ("embed_group_index", "biases[id * (K / 64) + k / 64]", "biases[id * (K / 64)]"),
    ("embed_out_of_range_zero", "            float v = NAN;", "            float v = 0.0f;"),
    ("i8g_one_scale_per_row", "(double)gs[m * (K / 64) + k / 64]", "(double)gs[m * (K / 64)]"),
    ("i8g_scales_transposed", "(double)gs[m * (K / 64) + k / 64]", "(double)gs[(k / 64) * A->M + m]"),
    ("i8g_group_of_128", "(double)gs[m * (K / 64) + k / 64]", "(double)gs[m * (K / 64) + k / 128]"),
    ("i8g_read_unsigned", "const int8_t *code = (const int8_t *)A->codes;",
     "const uint8_t *code = (const uint8_t *)A->codes;"),
    ("i8g_scale_dropped", "return (double)gs[m * (K / 64) + k / 64] * (double)code[m * K + k];",
     "(void)gs; return (double)code[m * K + k];"),
    # the sampled product (the reference of the large prefill cases)
    ("sample_n_m_swapped", "dot_one(&A, x, n_idx[i], m_idx[i], &y[i], &a[i]);",
     "dot_one(&A, x, m_idx[i], n_idx[i], &y[i], &a[i]);"),
    ("sample_x_by_output", "dot_one(&A, x, n_idx[i], m_idx[i], &y[i], &a[i]);",
     "dot_one(&A, x, m_idx[i], m_idx[i], &y[i], &a[i]);"),
    ("sample_outputs_reversed", "dot_one(&A, x, n_idx[i], m_idx[i], &y[i], &a[i]);",
     "dot_one(&A, x, n_idx[i], m_idx[i], &y[count - 1 - i], &a[count - 1 - i]);"),
    ("sample_first_pair_only", "dot_one(&A, x, n_idx[i], m_idx[i], &y[i], &a[i]);",
     "dot_one(&A, x, n_idx[0], m_idx[0], &y[i], &a[i]);"),
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = os.path.join(workdir, f"{name}.c")
    lib = os.path.join(workdir, f"lib{name}.so")
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", src, "-o", lib, "-lm"],
                   check=True)
    mutant = oracle.Oracle(lib)
    failed = []
    for pin in pins.PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
