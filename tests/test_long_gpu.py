"""Long sequences against the fp64 oracle, every element of every output
compared: T = 16384 and 8191 at head size 64 (the latter a ragged last
tile, 64 preprocess chunks, 128 backward steps for the first key block),
T = 6000 in fp16, T = 4097 at head size 128, T = 4096 at head size 32 and
with attention dropout, and the fp32 path at T = 4096 and 8192. The
kernels' loops, per-chunk statistics and placement run here far past the
T = 1024 .. 2048 of the model workloads. The bars are the usual ones (bf16
and fp16: max-abs 2e-2, mean-abs 5e-3; fp32: max-abs 1e-5); measured at
T = 16384: bf16 max-abs 6.5e-3 (O), fp32 at T = 8192: 3.4e-6 (dV)."""
from __future__ import annotations

import pytest

from causal_self_attention_amd.inputs import make_inputs
from tests.gpu_helpers import (announce, assert_parity, errors, run_gpu, run_gpu_dropout,
                               run_oracle, run_oracle_dropout)

pytestmark = pytest.mark.gpu

CASES = [("bf16", 1, 1, 16384, 64), ("bf16", 1, 2, 8191, 64), ("f16", 1, 1, 6000, 64),
         ("bf16", 1, 1, 4097, 128), ("bf16", 2, 1, 4096, 32), ("f32", 1, 1, 4096, 64),
         ("f32", 1, 1, 8192, 32)]


@pytest.mark.parametrize("dtype,B,H,T,D", CASES)
def test_long_sequence_full_compare(dtype, B, H, T, D):
    label = f"long dtype={dtype} B={B} H={H} T={T} D={D}"
    announce(label)
    inp = make_inputs(B, H, T, D, dtype, seed=T)
    assert_parity(errors(run_gpu(inp), run_oracle(inp)), dtype, label)


def test_long_sequence_with_dropout():
    drop = (0.1, 0x5EED5EED12345678, 3)
    label = "long dropout bf16 B=1 H=1 T=4096 D=64"
    announce(label)
    inp = make_inputs(1, 1, 4096, 64, "bf16", seed=4096)
    gpu = run_gpu_dropout(inp, drop)
    assert_parity(errors(gpu, run_oracle_dropout(inp, drop)), "bf16", label)
