"""The fp64 oracle and the C ABI's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

Two programs are built into a temporary directory and run:
  * the oracle (oracle/attn_oracle.c) with tests/sanitize/oracle_selfcheck.c,
    by gcc with -fsanitize=address,undefined (leak checking on): every
    oracle entry point on small shapes, plus exact facts and error statuses;
  * the C ABI (csrc/gpt_attn_abi.hip) with stand-in launchers
    (tests/sanitize/launch_stubs.cpp) and tests/sanitize/abi_driver.cpp, by
    hipcc with the sanitizers on the host code only (-Xarch_host): argument
    validation and the launch arguments of every entry point, no GPU needed.
Any sanitizer report aborts the program with a non-zero status.
"""
from __future__ import annotations

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(exe, env_extra):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_selfcheck")
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
                    "-std=c99", "-pthread", os.path.join(ROOT, "oracle", "attn_oracle.c"),
                    os.path.join(SAN, "oracle_selfcheck.c"), "-o", exe, "-lm"],
                   check=True, timeout=300)
    assert "oracle self-check ok" in _run(exe, {"ASAN_OPTIONS": "detect_leaks=1"})


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_c_abi_host_code_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "causal_self_attention_amd", "csrc")
    subprocess.run([HIPCC, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                    "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address,undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc, "-I", SAN, "-x", "hip",
                    os.path.join(csrc, "gpt_attn_abi.hip"), os.path.join(SAN, "launch_stubs.cpp"),
                    os.path.join(SAN, "abi_driver.cpp"), "-o", exe],
                   check=True, timeout=600, cwd=str(tmp_path))
    # The HIP runtime's own allocations outlive main: leak checking off.
    assert "ABI self-check ok" in _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
