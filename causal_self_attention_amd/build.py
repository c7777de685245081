"""Build the gfx950 attention library in-tree with hipcc.

Produces causal_self_attention_amd/libgptattn.so from every csrc/*.hip file.
Run as ``python -m causal_self_attention_amd.build``; it compiles every time
it is called.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libgptattn.so")
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


def build(verbose: bool = False, extra_flags: list[str] | None = None,
          out: str | None = None) -> str:
    out = out or LIB_PATH
    cmd = [HIPCC, *HIP_FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), *sources(), "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
