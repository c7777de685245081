"""The allocation-free backward (gpt_attn_bwd_noalloc) against the workspace
form (gpt_attn_bwd) through the C ABI: the same kernels on the same inputs,
so dK and dV must agree bit for bit and dQ to the order of its fp32 atomic
adds, and both must meet the oracle's bars. Two calls in a row, the second
on a smaller problem than the first, since every call on a GPU reuses that
GPU's one static scratch array."""
from __future__ import annotations

import pytest
import torch

import causal_self_attention_amd as gattn
from causal_self_attention_amd.inputs import make_inputs
from tests.gpu_helpers import announce, assert_parity, errors, run_oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _forward(inp):
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
    gattn.gpt_attn_fwd(q, k, v, o, lse)
    return q, k, v, do, o, lse


def _grads(q):
    return tuple(torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
                 for _ in range(3))


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 64), ("bf16", 128)])
def test_noalloc_equals_workspace_form_two_calls(dtype, D):
    for (B, H, T) in [(3, 12, 1024), (2, 3, 333)]:
        announce(f"noalloc dtype={dtype} D={D} B={B} H={H} T={T}")
        inp = make_inputs(B, H, T, D, dtype, seed=T)
        q, k, v, do, o, lse = _forward(inp)
        ws = torch.empty(gattn.gpt_attn_bwd_workspace_bytes(B, H, T, D) // 4,
                         dtype=torch.float32, device=DEV)
        ref = _grads(q)
        gattn.gpt_attn_bwd(q, k, v, o, do, lse, *ref, ws)
        out = _grads(q)
        gattn.gpt_attn_bwd_noalloc(q, k, v, o, do, lse, *out)
        torch.cuda.synchronize()
        assert torch.equal(out[1], ref[1]) and torch.equal(out[2], ref[2]), (B, H, T)
        d = float((out[0].double() - ref[0].double()).abs().max())
        assert d <= 1e-6 * max(1.0, float(ref[0].abs().max())), (B, H, T, d)
        gpu = {"o": o.cpu(), "lse": lse.cpu(), "dq": out[0].cpu(), "dk": out[1].cpu(),
               "dv": out[2].cpu()}
        assert_parity(errors(gpu, run_oracle(inp)), dtype, f"noalloc B={B} H={H} T={T}")


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    announce("noalloc too large")
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(1, 1, 8, dtype=torch.float32, device=DEV)
    g = torch.zeros(1, 1, 8, 64, dtype=torch.float32, device=DEV)
    lib = gattn.load_library()
    import ctypes
    P = ctypes.c_void_p(q.data_ptr())
    L, G = ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(g.data_ptr())
    # 64 x 64 x 1024 rows need 16.8 MB of workspace: rejected before any launch.
    assert lib.gpt_attn_bwd_noalloc(1, 64, 64, 1024, 64, P, P, P, P, P, L, G, G, G, None) == 7
    assert gattn.gpt_attn_bwd_workspace_bytes(64, 64, 1024, 64) > gattn.NOALLOC_SCRATCH_BYTES
