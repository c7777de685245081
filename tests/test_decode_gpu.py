"""GPU parity of the one-query decode path against the oracle.

Sampling feeds the sequence back one position at a time (generate(), page
"nanoGPT: a real GPT in two 300-line files", section 2 "How the code
works"); the newest query attends to the cached keys and values of every
position up to its own. Bars as elsewhere: fp32 max-abs 1e-5; bf16 max-abs
2e-2 and mean-abs 5e-3, on O and LSE.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import causal_self_attention_amd as gattn
import oracle
from causal_self_attention_amd.inputs import (DECODE_WORKLOADS, decode_inputs, make_decode_inputs,
                                              make_inputs)
from tests.gpu_helpers import TOL, announce

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, label, lengths=None):
    tol = TOL[dtype]
    o = o_gpu.double().cpu().numpy()
    lse = lse_gpu.double().cpu().numpy()
    if lengths is not None:  # empty sequences: O = 0 exactly, LSE = -inf
        empty = np.asarray(lengths) == 0
        assert not o[empty].any() and np.all(lse[empty] == -np.inf), label
        o, lse, o_ref, lse_ref = o[~empty], lse[~empty], o_ref[~empty], lse_ref[~empty]
    for name, g, r in (("o", o, o_ref), ("lse", lse, lse_ref)):
        if g.size == 0:
            continue
        d = np.abs(g - r)
        assert np.isfinite(g).all(), f"{label}: {name} not finite"
        assert d.max() <= tol["max"], f"{label}: {name} max-abs {d.max():.3e}"
        if tol["mean"] is not None:
            assert d.mean() <= tol["mean"], f"{label}: {name} mean-abs {d.mean():.3e}"


def _run(inp, ragged_on_gpu=True):
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    lengths = inp["lengths"].to(DEV) if ragged_on_gpu else None
    o, lse = gattn.attention_decode(q, k, v, lengths)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 64), ("f16", 64), ("bf16", 32),
                                     ("f32", 32), ("f16", 32), ("bf16", 128), ("f32", 128),
                                     ("f16", 128)])
@pytest.mark.parametrize("ragged", [False, True])
@pytest.mark.parametrize("B,H,L", [(1, 1, 1), (1, 2, 7), (2, 3, 129), (1, 1, 1000), (3, 2, 257),
                                   (5, 1, 128)])
def test_decode_parity(dtype, D, ragged, B, H, L):
    announce(f"decode dtype={dtype} D={D} ragged={ragged} B={B} H={H} L={L}")
    inp = make_decode_inputs(B, H, L, D, dtype, seed=L + B, ragged=ragged)
    o, lse = _run(inp)
    o_ref, lse_ref = oracle.attn_decode(inp["q"], inp["k"], inp["v"], inp["lengths"].numpy())
    _check(o, lse, o_ref, lse_ref, dtype, f"decode {dtype} D={D} B={B} H={H} L={L}")


@pytest.mark.parametrize("name", list(DECODE_WORKLOADS))
def test_decode_workload_full_size(name):
    w = DECODE_WORKLOADS[name]
    announce(f"decode workload {name}")
    inp = decode_inputs(w, seed=0)
    o, lse = _run(inp)
    o_ref, lse_ref = oracle.attn_decode(inp["q"], inp["k"], inp["v"], inp["lengths"].numpy())
    _check(o, lse, o_ref, lse_ref, w.dtype, name)


def test_decode_is_the_forward_last_row():
    """decode(q = Q[T-1], caches = K, V) is the causal forward's row T-1."""
    B, H, T = 2, 3, 300
    announce(f"decode vs forward last row B={B} H={H} T={T}")
    inp = make_inputs(B, H, T, 64, "bf16", seed=9)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o_full, lse_full, _ = gattn.attention_forward(q, k, v)
    o, lse = gattn.attention_decode(q[:, :, -1].contiguous(), k, v)
    torch.cuda.synchronize()
    assert (o.float() - o_full[:, :, -1].float()).abs().max().item() <= 2e-2
    assert (lse - lse_full[:, :, -1]).abs().max().item() <= 1e-4


def test_decode_zero_lengths_and_empty_cache():
    announce("decode zero lengths / L = 0")
    inp = make_decode_inputs(3, 2, 50, 64, "bf16", seed=1)
    inp["lengths"] = torch.tensor([0, 50, 0], dtype=torch.int32)
    o, lse = _run(inp)
    o_ref, lse_ref = oracle.attn_decode(inp["q"], inp["k"], inp["v"], inp["lengths"].numpy())
    _check(o, lse, o_ref, lse_ref, "bf16", "zero lengths", lengths=[0, 50, 0])
    q = torch.randn(2, 2, 64, device=DEV).to(torch.bfloat16)
    kv = torch.empty(2, 2, 0, 64, dtype=torch.bfloat16, device=DEV)
    o, lse = gattn.attention_decode(q, kv, kv)
    torch.cuda.synchronize()
    assert not o.float().any() and bool((lse == -float("inf")).all())


def test_decode_ignores_rows_past_length_and_strided_cache():
    """Cache in [B, L, H, D] order (a token-major cache) with NaN in every row
    at or past each sequence's length."""
    B, H, L, D = 4, 3, 200, 64
    announce(f"decode strided cache B={B} H={H} L={L}")
    inp = make_decode_inputs(B, H, L, D, "bf16", seed=5, ragged=True)
    kbuf = torch.full((B, L, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    vbuf = torch.full((B, L, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lens = inp["lengths"].tolist()
    for b, n in enumerate(lens):
        kbuf[b, :n] = inp["k"][b, :, :n].transpose(0, 1).to(DEV)
        vbuf[b, :n] = inp["v"][b, :, :n].transpose(0, 1).to(DEV)
    k, v = kbuf.transpose(1, 2), vbuf.transpose(1, 2)  # [B, H, L, D] views
    obuf = torch.full((B, H, D + 8), 1024.0, dtype=torch.bfloat16, device=DEV)
    o, lse = gattn.attention_decode(inp["q"].to(DEV), k, v, inp["lengths"].to(DEV),
                                    out=obuf[:, :, :D])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_decode(inp["q"], inp["k"], inp["v"], lens)
    _check(o, lse, o_ref, lse_ref, "bf16", "strided cache")
    assert bool((obuf[:, :, D:].float() == 1024.0).all())
