"""GPU parity at head dimension 128.

D = 128 runs its own backward: a dK/dV kernel (32 keys per wave, one wave
per SIMD) and a dQ kernel (32 queries per wave, dQ written once, no
atomics), after the same preprocess; the forward is the D = 32/64 kernel
with each 64-key tile taken half by half. Each case runs forward + backward
through the C ABI and compares every output element with the fp64 oracle on
the same inputs at the usual bars.
"""
from __future__ import annotations

import pytest
import torch

from causal_self_attention_amd.inputs import make_inputs
from tests.gpu_helpers import (announce, assert_parity, errors, run_gpu, run_gpu_dropout,
                               run_oracle, run_oracle_dropout)

pytestmark = pytest.mark.gpu

D = 128


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 64, 65, 127, 128, 129, 200, 255, 256, 257, 300])
def test_small_shapes(dtype, T):
    announce(f"D=128 parity dtype={dtype} T={T}")
    inp = make_inputs(1, 3, T, D, dtype, seed=1280 + T)
    assert_parity(errors(run_gpu(inp), run_oracle(inp)), dtype, f"D=128 {dtype} T={T}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,H,T", [(2, 3, 515), (1, 5, 1000)])
def test_with_o_lo(dtype, B, H, T):
    announce(f"D=128 o_lo dtype={dtype} B={B} H={H} T={T}")
    inp = make_inputs(B, H, T, D, dtype, seed=1290 + T)
    assert_parity(errors(run_gpu(inp, o_lo=True), run_oracle(inp)), dtype,
                  f"D=128 o_lo {dtype} T={T}")


@pytest.mark.parametrize("dtype,T,p", [("bf16", 77, 0.1), ("bf16", 333, 0.2), ("f16", 300, 0.2),
                                       ("f32", 150, 0.3)])
def test_dropout(dtype, T, p):
    drop = (p, 1234 + T, 7)
    announce(f"D=128 dropout dtype={dtype} T={T} drop={drop}")
    inp = make_inputs(2, 2, T, D, dtype, seed=1300 + T)
    assert_parity(errors(run_gpu_dropout(inp, drop), run_oracle_dropout(inp, drop)), dtype,
                  f"D=128 dropout {dtype} T={T} p={p}")


def test_backward_is_reproducible():
    """No atomics at D = 128: dQ, dK and dV are bitwise equal run to run."""
    announce("D=128 determinism")
    inp = make_inputs(2, 3, 700, D, "bf16", seed=1310)
    a, b = run_gpu(inp), run_gpu(inp)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("name,k", [("do", -20), ("do", 16), ("v", -16), ("v", 20), ("qk", -16)])
def test_scaled_inputs(name, k):
    """One input times 2^k (bf16, exact): errors divided by the factor each
    output scales by stay within the bars (see test_range_gpu)."""
    announce(f"D=128 range {name} x 2^{k}")
    inp = make_inputs(2, 2, 333, D, "bf16", seed=1320)
    names = {"do": ("do",), "v": ("v",), "qk": ("q", "k")}[name]
    exps = {"do": {"o": 0, "lse": 0, "dq": 1, "dk": 1, "dv": 1},
            "v": {"o": 1, "lse": 0, "dq": 1, "dk": 1, "dv": 0},
            "qk": {"o": 0, "lse": 0, "dq": 1, "dk": 1, "dv": 0}}[name]
    for n in names:
        inp[n] = (inp[n].float() * 2.0 ** k).to(torch.bfloat16)
    gpu, ref = run_gpu(inp), run_oracle(inp)
    scaled = {n: (gpu[n].double() / 2.0 ** (k * e)) for n, e in exps.items()}
    ref_s = {n: ref[n] / 2.0 ** (k * e) for n, e in exps.items()}
    assert_parity(errors(scaled, ref_s), "bf16", f"D=128 {name} x 2^{k}")
