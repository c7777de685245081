"""GPU parity of attention dropout against the oracle.

nanoGPT trains with its dropout rate handed to the fused attention call
(page "nanoGPT: a real GPT in two 300-line files", section 2 "How the code
works"); its Shakespeare-char configuration uses 0.2 (section 3 "Run it,
tested"). The kernels regenerate a Philox4x32-10 keep mask; the oracle
derives the same mask independently and runs attention with it explicitly.
The mask itself is integer work and must match bit for bit; the attention
outputs meet the usual bars (fp32 max-abs 1e-5; bf16 max-abs 2e-2 and
mean-abs 5e-3).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import causal_self_attention_amd as gattn
import oracle
from causal_self_attention_amd.inputs import WORKLOADS, make_inputs, workload_inputs
from tests.gpu_helpers import (announce, assert_parity, errors, run_gpu, run_gpu_dropout,
                               run_oracle_dropout)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.mark.parametrize("B,H,T,p,seed,offset", [
    (1, 1, 1, 0.2, 0, 0), (1, 2, 13, 0.2, 1, 0), (2, 3, 100, 0.5, 2**64 - 1, 7),
    (1, 1, 257, 0.1, 0x1234_5678_9ABC_DEF0, 2**32 - 1), (3, 2, 64, 0.99999, 42, 3),
    (1, 1, 33, 0.0, 5, 5)])
def test_keep_mask_bit_exact(B, H, T, p, seed, offset):
    announce(f"dropout mask B={B} H={H} T={T} p={p} seed={seed} offset={offset}")
    mask = torch.full((B, H, T, T), 7, dtype=torch.uint8, device=DEV)
    gattn.gpt_attn_dropout_mask(B, H, T, (p, seed, offset), mask)
    torch.cuda.synchronize()
    ref = oracle.dropout_keep(range(B * H), T, p, seed, offset).reshape(B, H, T, T)
    got = mask.cpu().numpy()
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} entries differ"


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 64), ("f16", 64), ("bf16", 32),
                                     ("f32", 32)])
@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (1, 1, 31), (1, 2, 65), (2, 3, 333), (1, 1, 300)])
def test_dropout_parity(dtype, D, B, H, T):
    drop = (0.2, 1000 + T, 3)
    announce(f"dropout parity dtype={dtype} D={D} B={B} H={H} T={T} drop={drop}")
    inp = make_inputs(B, H, T, D, dtype, seed=T + 50)
    gpu = run_gpu_dropout(inp, drop)
    ref = run_oracle_dropout(inp, drop)
    assert_parity(errors(gpu, ref), dtype, f"dropout {dtype} D={D} B={B} H={H} T={T}")


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_dropout_rates(p):
    """The survivor scale z = 1/(1-p) multiplies O and the gradients, and with
    them the bf16 rounding of the outputs; the bars are for unit-scale
    attention, so they apply to the errors divided by z (z = 10 at p = 0.9;
    at p <= 0.5 the plain bars hold as well)."""
    drop = (p, 99, 1)
    announce(f"dropout rate p={p} bf16 B=1 H=2 T=200")
    inp = make_inputs(1, 2, 200, 64, "bf16", seed=7)
    errs = errors(run_gpu_dropout(inp, drop), run_oracle_dropout(inp, drop))
    z = oracle.dropout_scale(p)
    assert_parity({n: (mx / z, mean / z) for n, (mx, mean) in errs.items()}, "bf16", f"p={p}")
    if p <= 0.5:
        assert_parity(errs, "bf16", f"p={p} unscaled")


def test_dropout_shakespeare_char_full_size():
    """The Shakespeare-char "baby GPT" attention layer (B=64, H=6, T=256) at
    the dropout it trains with (0.2), bf16: sampled heads against the oracle."""
    w = WORKLOADS["shakespeare_char_bf16_b64_h6_t256"]
    drop = (0.2, 1337, 0)
    announce(f"dropout full size {w.name} drop={drop}")
    inp = workload_inputs(w, seed=0)
    gpu = run_gpu_dropout(inp, drop)
    heads = [0, 37, 190, w.B * w.H - 1]
    ref = run_oracle_dropout(inp, drop, heads)
    assert_parity(errors(gpu, ref, heads), "bf16", f"dropout {w.name} heads {heads}")


def test_dropout_shakespeare_char_f32():
    w = WORKLOADS["shakespeare_char_f32_b1_h6_t256"]
    drop = (0.2, 2024, 11)
    announce(f"dropout full size {w.name} drop={drop}")
    inp = workload_inputs(w, seed=0)
    assert_parity(errors(run_gpu_dropout(inp, drop), run_oracle_dropout(inp, drop)), "f32",
                  w.name)


def test_p_zero_is_the_plain_path():
    inp = make_inputs(2, 2, 150, 64, "bf16", seed=3)
    announce("dropout p=0 equals no dropout")
    a = run_gpu_dropout(inp, (0.0, 5, 5))
    b = run_gpu(inp, o_lo=True)
    for n in ("o", "lse", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n
    assert (a["dq"] - b["dq"]).abs().max().item() <= 1e-5


def test_dropout_streams_and_determinism():
    inp = make_inputs(1, 2, 120, 64, "bf16", seed=4)
    announce("dropout determinism and streams")
    a = run_gpu_dropout(inp, (0.3, 10, 0))
    b = run_gpu_dropout(inp, (0.3, 10, 0))
    c = run_gpu_dropout(inp, (0.3, 10, 1))
    for n in ("o", "lse", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n
    assert torch.equal(a["lse"], c["lse"])          # the softmax ignores dropout
    assert not torch.equal(a["o"], c["o"])          # another stream, another mask


def test_dropout_with_fused_layout():
    """Dropout through the strided calls on the projection layout."""
    B, H, T, D = 2, 3, 190, 64
    drop = (0.2, 77, 2)
    announce(f"dropout fused layout B={B} H={H} T={T}")
    inp = make_inputs(B, H, T, D, "bf16", seed=12)
    C = H * D
    qkv = torch.empty(B, T, 3 * C, dtype=torch.bfloat16, device=DEV)
    q, k, v = gattn.split_qkv_heads(qkv, H)
    for view, name in ((q, "q"), (k, "k"), (v, "v")):
        view.copy_(inp[name].to(DEV))
    do = gattn.merged_heads_view(torch.empty(B, T, C, dtype=torch.bfloat16, device=DEV), H)
    do.copy_(inp["do"].to(DEV))
    o = gattn.merged_heads_view(torch.empty(B, T, C, dtype=torch.bfloat16, device=DEV), H)
    g = torch.empty(B, T, 3 * C, dtype=torch.float32, device=DEV)
    dq, dk, dv = gattn.split_qkv_heads(g, H)
    _, lse, o_lo = gattn.attention_forward(q, k, v, out=o, dropout=drop)
    gattn.attention_backward(q, k, v, o, do, lse, o_lo, grads=(dq, dk, dv), dropout=drop)
    torch.cuda.synchronize()
    gpu = {"o": o.contiguous().cpu(), "lse": lse.cpu(), "dq": dq.contiguous().cpu(),
           "dk": dk.contiguous().cpu(), "dv": dv.contiguous().cpu()}
    assert_parity(errors(gpu, run_oracle_dropout(inp, drop)), "bf16", "dropout fused layout")
