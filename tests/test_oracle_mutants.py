"""Planted mistakes in the oracle must be caught by its pins.

Each case copies attn_oracle.c, plants one plausible mistake (a dropped term,
a wrong sign, a wrong index, a transposed operand, a shifted mask), compiles
the copy on the CPU into a temporary library, swaps it in for the real one and
runs the pins of test_oracle_pins. At least one pin must fail for every
mutant; the real oracle must pass them all.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

# (name, original text, planted text). Every original must occur in the source.
MUTANTS = [
    ("scale_dropped", "const double s = 1.0 / sqrt((double)D);", "const double s = 1.0;"),
    ("diagonal_masked", "for (long j = 0; j <= i; ++j) {\n    const double* kj = k + j * D;\n    double dot",
     "for (long j = 0; j < i; ++j) {\n    const double* kj = k + j * D;\n    double dot"),
    ("max_not_subtracted_in_lse", "return m + log(l);", "return log(l);"),
    ("ds_sign", "p[j] * (dp - delta[i]);\n      double* dvj", "p[j] * (dp + delta[i]);\n      double* dvj"),
    ("dk_transposed_operand", "dkj[d] += s * ds * qi[d];", "dkj[d] += s * ds * kj[d];"),
    ("dq_wrong_operand", "dqi[d] += s * ds * kj[d];", "dqi[d] += s * ds * vj[d];"),
    ("dv_dropped_weight", "dvj[d] += p[j] * doi[d];", "dvj[d] += doi[d];"),
    ("delta_from_v", "acc += dout[i * D + d] * o[i * D + d];\n    delta[i] = acc;\n  }\n  memset(dq",
     "acc += dout[i * D + d] * v[i * D + d];\n    delta[i] = acc;\n  }\n  memset(dq"),
    ("dq_scale_dropped", "dqi[d] += s * ds * kj[d];", "dqi[d] += ds * kj[d];"),
    ("output_row_offset", "double* oi = o + i * D;", "double* oi = o + (i > 0 ? i - 1 : 0) * D;"),
]


# Planted mistakes in the dropout half of the oracle (generator, mask mapping,
# threshold, forward and backward with a mask).
DROPOUT_MUTANTS = [
    ("philox_lo_words_swapped", "const uint32_t y1 = (uint32_t)p1;", "const uint32_t y1 = (uint32_t)p0;"),
    ("philox_no_key_bump", "    k0 += W0;\n    k1 += W1;\n  }", "    k1 += W1;\n  }"),
    ("philox_nine_rounds", "for (int r = 0; r < 10; ++r) {\n    const uint64_t p0",
     "for (int r = 0; r < 9; ++r) {\n    const uint64_t p0"),
    ("mask_counter_words_swapped", "{(uint32_t)(j / 8), (uint32_t)i, (uint32_t)bh[h], offset}",
     "{(uint32_t)i, (uint32_t)(j / 8), (uint32_t)bh[h], offset}"),
    ("mask_word_index", "out[(j % 8) / 2]", "out[(j % 4)]"),
    ("mask_field", "(16 * (j % 2))", "(16 * ((j / 2) % 2))"),
    ("threshold_truncated", "floor(p * 65536.0 + 0.5)", "floor(p * 65536.0)"),
    ("keep_compare_strict", "u >= (uint32_t)thr ? 1 : 0", "u > (uint32_t)thr ? 1 : 0"),
    ("fwd_scale_missing", "const double pd = M[i * T + j] ? z * p[j] : 0.0;\n      const double* vj",
     "const double pd = M[i * T + j] ? p[j] : 0.0;\n      const double* vj"),
    ("bwd_mask_ignored_in_dp", "dp[j] = M[i * T + j] ? z * dpd : 0.0;", "dp[j] = z * dpd;"),
    ("bwd_dv_undropped", "const double pd = M[i * T + j] ? z * p[j] : 0.0;\n      double* dvj",
     "const double pd = p[j];\n      double* dvj"),
    ("bwd_rowdot_undropped", "rowdot += p[j] * dp[j];", "rowdot += p[j] * dpd;"),
]


# Planted mistakes in the one-query decode function.
DECODE_MUTANTS = [
    ("decode_length_off_by_one", "for (long j = 0; j < n; ++j) {\n      double dot",
     "for (long j = 0; j + 1 < n; ++j) {\n      double dot"),
    ("decode_unnormalized", "oh[d] += (p[j] / l) * vh[j * D + d];", "oh[d] += p[j] * vh[j * D + d];"),
    ("decode_lse_without_max", "lse[h] = m + log(l);\n  }\n  free(p);", "lse[h] = log(l);\n  }\n  free(p);"),
    ("decode_cache_stride", "const double* kh = k + h * L * D;", "const double* kh = k + h * D;"),
]


def _decode_pin_suite():
    from tests import test_oracle_decode as dc
    return [
        ("last_row", lambda: dc.test_equals_last_row_of_causal_forward(17, 8)),
        ("brute", lambda: dc.test_brute_force_last_row(6, 5)),
        ("closed", dc.test_closed_forms),
        ("lengths", dc.test_rows_past_length_are_ignored_and_lengths_per_head),
    ]


def _dropout_pin_suite(rocrand_ref):
    from tests import test_oracle_dropout as dp
    suite = [
        ("thresholds", dp.test_threshold_values),
        ("statistics", dp.test_mask_statistics),
        ("keep_all", dp.test_keep_all_equals_plain_oracle),
        ("closed_forms", dp.test_closed_forms_all_dropped_and_diagonal_only),
        ("fd", lambda: dp.test_finite_differences_with_mask((1, 1, 6, 3))),
        ("brute", lambda: dp.test_brute_force_decimal_with_mask((1, 2, 5, 3))),
    ]
    if rocrand_ref is not None:
        suite += [("rocrand_blocks", lambda: dp.test_philox_matches_rocrand(rocrand_ref)),
                  ("rocrand_mask", lambda: dp.test_keep_mask_recomputed_from_rocrand(rocrand_ref)),
                  ("boundary", lambda: dp.test_threshold_compare_boundary(rocrand_ref))]
    return suite


def _pin_suite():
    """(name, callable) for every pin in test_oracle_pins."""
    suite = []
    for ex in pins._golden_examples():
        suite.append((f"fixture:{ex['name']}", lambda ex=ex: pins.test_closed_form_fixture(ex)))
    for shape in [(1, 2, 5, 3), (1, 1, 9, 12)]:
        suite.append((f"brute:{shape}", lambda s=shape: pins.test_brute_force_decimal(s)))
    suite.append(("fd", lambda: pins.test_central_finite_differences((1, 1, 5, 3))))
    suite.append(("sdpa", lambda: pins.test_matches_torch_sdpa_fp64((2, 3, 37, 16))))
    suite.append(("row0", pins.test_row_zero_exact))
    suite.append(("t1", pins.test_single_position))
    suite.append(("uniform_k", lambda: pins.test_uniform_attention(False)))
    suite.append(("uniform_q", lambda: pins.test_uniform_attention(True)))
    suite.append(("row_sums", pins.test_probability_rows_and_zero_score_gradient_rows))
    suite.append(("col_sums", pins.test_column_sums))
    suite.append(("value_affine", pins.test_value_affine_equivariance))
    suite.append(("key_shift", pins.test_key_shift))
    return suite


@contextlib.contextmanager
def _swapped_oracle(lib_path):
    saved = oracle._lib
    oracle._lib = None
    saved_path = oracle._LIB_PATH
    oracle._LIB_PATH = lib_path
    try:
        oracle._load()
        yield
    finally:
        oracle._lib = saved
        oracle._LIB_PATH = saved_path


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)  # the first site: the plain half precedes dropout
    c_path = tmp_path / f"{name}.c"
    c_path.write_text(mutated)
    so_path = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c99", "-shared",
                    "-fPIC", "-pthread", str(c_path), "-o", str(so_path), "-lm"], check=True)
    return str(so_path)


def _failing_pins(suite=None):
    failed = []
    for pin_name, fn in (suite if suite is not None else _pin_suite()):
        try:
            fn()
        except (AssertionError, ValueError):
            failed.append(pin_name)
    return failed


def test_real_oracle_passes_every_pin():
    assert _failing_pins() == []


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    from tests import test_oracle_dropout as dp
    return dp.build_rocrand_ref(tmp_path_factory.mktemp("rocrand_mut"))


def test_real_oracle_passes_every_dropout_pin(rocrand_ref):
    assert rocrand_ref is not None, "hipcc / rocRAND headers missing"
    assert _failing_pins(_dropout_pin_suite(rocrand_ref)) == []


@pytest.mark.parametrize("name,old,new", DROPOUT_MUTANTS, ids=[m[0] for m in DROPOUT_MUTANTS])
def test_dropout_mutant_is_caught(tmp_path, rocrand_ref, name, old, new):
    lib = _build_mutant(tmp_path, name, old, new)
    with _swapped_oracle(lib):
        failed = _failing_pins(_dropout_pin_suite(rocrand_ref))
    assert failed, f"no pin caught the planted mistake {name}"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    lib = _build_mutant(tmp_path, name, old, new)
    with _swapped_oracle(lib):
        failed = _failing_pins()
    assert failed, f"no pin caught the planted mistake {name}"


def test_real_oracle_passes_every_decode_pin():
    assert _failing_pins(_decode_pin_suite()) == []


@pytest.mark.parametrize("name,old,new", DECODE_MUTANTS, ids=[m[0] for m in DECODE_MUTANTS])
def test_decode_mutant_is_caught(tmp_path, name, old, new):
    lib = _build_mutant(tmp_path, name, old, new)
    with _swapped_oracle(lib):
        failed = _failing_pins(_decode_pin_suite())
    assert failed, f"no pin caught the planted mistake {name}"
