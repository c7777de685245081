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
    mutated = src.replace(old, new)
    c_path = tmp_path / f"{name}.c"
    c_path.write_text(mutated)
    so_path = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c99", "-shared",
                    "-fPIC", "-pthread", str(c_path), "-o", str(so_path), "-lm"], check=True)
    return str(so_path)


def _failing_pins():
    failed = []
    for pin_name, fn in _pin_suite():
        try:
            fn()
        except AssertionError:
            failed.append(pin_name)
    return failed


def test_real_oracle_passes_every_pin():
    assert _failing_pins() == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    lib = _build_mutant(tmp_path, name, old, new)
    with _swapped_oracle(lib):
        failed = _failing_pins()
    assert failed, f"no pin caught the planted mistake {name}"
