"""The forward and backward captured in a HIP graph (how the benchmark times
a step) give, on every replay, what eager launches give: replays run with
the program's own eager work and synchronizations in between, and each one
is checked (O, LSE, dK, dV bit for bit; dQ to atomics rounding)."""
from __future__ import annotations

import pytest
import torch

import causal_self_attention_amd as gattn
from causal_self_attention_amd.inputs import make_inputs
from tests.gpu_helpers import announce

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.mark.parametrize("dropout", [None, (0.2, 7, 1)])
def test_graph_replays_match_eager(dropout):
    B, H, T = 2, 3, 300
    announce(f"graph replay B={B} H={H} T={T} dropout={dropout}")
    inp = make_inputs(B, H, T, 64, "bf16", seed=41)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    o_lo = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
    dq = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    ws = torch.empty(gattn.gpt_attn_bwd_workspace_bytes(B, H, T, 64) // 4, dtype=torch.float32,
                     device=DEV)

    def step():
        st = torch.cuda.current_stream(DEV)
        gattn.gpt_attn_fwd_strided(q, k, v, o, o_lo, lse, st, dropout)
        gattn.gpt_attn_bwd_prep_strided(q, o, o_lo, do, dq, ws, st)
        gattn.gpt_attn_bwd_main_strided(q, k, v, do, lse, dq, dk, dv, ws, st, dropout)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]

    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    other = make_inputs(1, 2, 77, 64, "bf16", seed=3)
    for rep in range(4):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        # Eager work of the program between replays.
        gattn.attention_forward(*(other[n].to(DEV) for n in ("q", "k", "v")))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
            if name == "dq":
                assert (got - want).abs().max().item() <= 1e-5, (rep, name)
            else:
                assert torch.equal(got, want), (rep, name)
