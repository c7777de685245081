"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and compare with the fp64 oracle on identical seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import causal_self_attention_amd as gattn
import oracle

# Tolerances of the parity bar, per output tensor (O, LSE, dQ, dK, dV):
# fp32 inputs: max-abs error <= 1e-5; bf16 inputs (fp32 accumulation):
# max-abs <= 2e-2 and mean-abs <= 5e-3.
# fp16 inputs (11-bit significands) are held to the bf16 bars.
TOL = {"f32": {"max": 1e-5, "mean": None}, "bf16": {"max": 2e-2, "mean": 5e-3},
       "f16": {"max": 2e-2, "mean": 5e-3}}


def announce(msg: str) -> None:
    """Name the case on stderr (past pytest's capture) before a GPU step."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def run_gpu(inp: dict, o_lo: bool = False):
    """Forward + backward on cuda:0 through the C ABI. Returns CPU tensors
    o, lse, dq, dk, dv. By default the plain entry points (gpt_attn_fwd,
    gpt_attn_bwd); with ``o_lo`` the strided ones with the forward's low
    part of O passed to the backward."""
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    if o_lo:
        o, lse, lo = gattn.attention_forward(q, k, v, keep_o_lo=True)
        dq, dk, dv = gattn.attention_backward(q, k, v, o, do, lse, lo)
    else:
        B, H, T, D = q.shape
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
        ws = torch.empty(max(1, gattn.gpt_attn_bwd_workspace_bytes(B, H, T, D) // 4),
                         dtype=torch.float32, device=dev)
        gattn.gpt_attn_fwd(q, k, v, o, lse)
        gattn.gpt_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}


def run_oracle(inp: dict, heads=None):
    """fp64 oracle on the same (already dtype-rounded) inputs. ``heads`` is an
    optional list of flat head indices to restrict the work to."""
    arrs = {n: inp[n].double().numpy() for n in ("q", "k", "v", "do")}
    B, H, T, D = arrs["q"].shape
    if heads is not None:
        arrs = {n: a.reshape(B * H, T, D)[heads] for n, a in arrs.items()}
    o, lse = oracle.attn_fwd(arrs["q"], arrs["k"], arrs["v"])
    dq, dk, dv = oracle.attn_bwd(arrs["q"], arrs["k"], arrs["v"], arrs["do"])
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def errors(gpu: dict, ref: dict, heads=None) -> dict:
    out = {}
    for name, r in ref.items():
        g = gpu[name].double().numpy()
        if heads is not None:
            g = g.reshape((-1,) + g.shape[2:])[heads]
        d = np.abs(g - r)
        out[name] = (float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0)
    return out


def assert_parity(errs: dict, dtype: str, label: str) -> None:
    tol = TOL[dtype]
    bad = []
    for name, (mx, mean) in errs.items():
        if mx > tol["max"] or not np.isfinite(mx):
            bad.append(f"{name}: max-abs {mx:.3e} > {tol['max']}")
        if tol["mean"] is not None and mean > tol["mean"]:
            bad.append(f"{name}: mean-abs {mean:.3e} > {tol['mean']}")
    assert not bad, f"{label}: " + "; ".join(bad)


def run_gpu_dropout(inp: dict, dropout, keep_o_lo: bool = True):
    """run_gpu with attention dropout ``dropout`` = (p, seed, offset)."""
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse, o_lo = gattn.attention_forward(q, k, v, keep_o_lo=keep_o_lo, dropout=dropout)
    dq, dk, dv = gattn.attention_backward(q, k, v, o, do, lse, o_lo, dropout=dropout)
    torch.cuda.synchronize()
    return {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}


def run_oracle_dropout(inp: dict, dropout, heads=None):
    """fp64 oracle with the keep mask the oracle derives for ``dropout``."""
    p, seed, offset = dropout
    arrs = {n: inp[n].double().numpy() for n in ("q", "k", "v", "do")}
    B, H, T, D = arrs["q"].shape
    flat = list(range(B * H)) if heads is None else list(heads)
    arrs = {n: a.reshape(B * H, T, D)[flat] for n, a in arrs.items()}
    keep = oracle.dropout_keep(flat, T, p, seed, offset)
    z = oracle.dropout_scale(p)
    o, lse = oracle.attn_fwd_dropout(arrs["q"], arrs["k"], arrs["v"], keep, z)
    dq, dk, dv = oracle.attn_bwd_dropout(arrs["q"], arrs["k"], arrs["v"], arrs["do"], keep, z)
    if heads is None:
        shape = (B, H, T, D)
        o, dq, dk, dv = (x.reshape(shape) for x in (o, dq, dk, dv))
        lse = lse.reshape(B, H, T)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
