"""Build the gfx950 attention library in-tree with hipcc.

Produces causal_self_attention_amd/libgptattn.so from every csrc/*.hip file,
and libgptattn_dbg.so, the same sources with GPT_ATTN_EXTRA_BARRIERS (a
full workgroup barrier at every marked LDS stage boundary; the race check
of the test suite compares its results with the release library's), and
libsclkprobe.so from probe/sclk_probe.hip (the benchmark's shader-clock
probe; not part of the attention library). Run as
``python -m causal_self_attention_amd.build``; it compiles every time it is
called.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libgptattn.so")
DBG_LIB_PATH = os.path.join(HERE, "libgptattn_dbg.so")
PROBE_LIB_PATH = os.path.join(HERE, "libsclkprobe.so")
PROBE_SOURCE = os.path.join(HERE, "probe", "sclk_probe.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU instructions stay off: the compiler is told the target
# lacks them, so ordinary float code is emitted as scalar VALU operations.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _command(out: str, extra_flags: list[str] | None, srcs: list[str] | None = None) -> list[str]:
    return [HIPCC, *HIP_FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(HERE, "csrc"), *(srcs or sources()), "-o", out + ".tmp"]


def build(verbose: bool = False, extra_flags: list[str] | None = None,
          out: str | None = None, debug_too: bool = True) -> str:
    """Build libgptattn.so (and, unless debug_too is false, libgptattn_dbg.so
    alongside it, the two compilations running at once)."""
    out = out or LIB_PATH
    jobs = [(out, extra_flags, None)]
    if debug_too and out == LIB_PATH:
        jobs.append((DBG_LIB_PATH, [*(extra_flags or []), "-DGPT_ATTN_EXTRA_BARRIERS"], None))
        jobs.append((PROBE_LIB_PATH, None, [PROBE_SOURCE]))
    procs = []
    for path, flags, srcs in jobs:
        cmd = _command(path, flags, srcs)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((path, subprocess.Popen(cmd)))
    failed = [path for path, p in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, f"hipcc for {', '.join(failed)}")
    for path, _ in procs:
        os.replace(path + ".tmp", path)
    return out


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
