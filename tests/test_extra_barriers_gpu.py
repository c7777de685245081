"""Race check of the LDS pipelines: the library built with
GPT_ATTN_EXTRA_BARRIERS (libgptattn_dbg.so, a full workgroup barrier at every
marked LDS stage boundary, so no two stages overlap) must give the release
library's results bit for bit: O, LSE, dK and dV exactly, dQ to the order of
its fp32 atomic adds. A missing wait in the release schedule (a tile read
while the next one is written, a dS buffer reused too early) would show up
as a difference."""
from __future__ import annotations

import ctypes
import os

import pytest
import torch

import causal_self_attention_amd as gattn
from causal_self_attention_amd.inputs import make_inputs
from tests.gpu_helpers import announce

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
DBG_PATH = os.path.join(os.path.dirname(gattn.library_path()), "libgptattn_dbg.so")


def _debug_library():
    if not os.path.exists(DBG_PATH):
        raise RuntimeError(f"{DBG_PATH} is not built; run `python -m causal_self_attention_amd.build`")
    rel = gattn.load_library()
    dbg = ctypes.CDLL(DBG_PATH)
    for name in ("gpt_attn_fwd_strided", "gpt_attn_bwd_strided", "gpt_attn_abi_version"):
        f, g = getattr(rel, name), getattr(dbg, name)
        g.argtypes, g.restype = f.argtypes, f.restype
    assert dbg.gpt_attn_abi_version() == rel.gpt_attn_abi_version()
    return rel, dbg


def _run(lib, inp, dropout, o_lo):
    """Forward + backward through lib's strided entry points (contiguous
    layouts); returns CPU copies of o, lse, dq, dk, dv."""
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    B, H, T, D = q.shape
    code = gattn._dtype_code(q)
    o = torch.empty_like(q)
    lo = torch.empty_like(q) if o_lo else None
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=DEV) for _ in range(3))
    ws = torch.empty(gattn.gpt_attn_bwd_workspace_bytes(B, H, T, D) // 4, dtype=torch.float32,
                     device=DEV)
    p = gattn._ptr
    drop = gattn._dropout_arg(dropout)
    st = gattn._stream(DEV, None)
    assert lib.gpt_attn_fwd_strided(code, B, H, T, D, p(q), None, p(k), None, p(v), None, p(o),
                                    None, p(lo), None, p(lse), drop, st) == 0
    assert lib.gpt_attn_bwd_strided(code, B, H, T, D, p(q), None, p(k), None, p(v), None, p(o),
                                    None, p(lo), None, p(do), None, p(lse), p(dq), None, p(dk),
                                    None, p(dv), None, p(ws), ws.numel() * 4, drop, st) == 0
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}


CASES = [("bf16", 64, 1000, None, False), ("bf16", 64, 333, (0.2, 11, 3), True),
         ("f16", 64, 515, None, True), ("bf16", 32, 300, None, False),
         ("f16", 32, 129, (0.1, 5, 0), False), ("f32", 64, 300, None, False),
         ("f32", 32, 77, (0.3, 9, 1), False), ("bf16", 64, 1000, "growing_v", False),
         ("bf16", 128, 700, None, True), ("f16", 128, 257, (0.2, 3, 4), False)]


@pytest.mark.parametrize("dtype,D,T,dropout,o_lo", CASES)
def test_extra_barrier_build_matches_release(dtype, D, T, dropout, o_lo):
    announce(f"extra barriers dtype={dtype} D={D} T={T} dropout={dropout} o_lo={o_lo}")
    rel, dbg = _debug_library()
    inp = make_inputs(2, 3, T, D, dtype, seed=500 + T)
    if dropout == "growing_v":
        # V doubling every 64 keys: the forward's V exponent moves mid-sequence.
        f = (2.0 ** (torch.arange(T) // 64).double()).view(1, 1, T, 1)
        inp["v"] = (inp["v"].double() * f).to(inp["v"].dtype)
        dropout = None
    a = _run(rel, inp, dropout, o_lo)
    b = _run(dbg, inp, dropout, o_lo)
    for n in ("o", "lse", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n
    d = float((a["dq"].double() - b["dq"].double()).abs().max())
    assert d <= 1e-6 * max(1.0, float(a["dq"].abs().max())), d
