"""GPU parity of the strided entry points.

The attention layer makes q, k, v for every token with one linear map and
splits them into heads; the merged head outputs feed the next projection
(page "nanoGPT: a real GPT in two 300-line files", section 2 "How the code
works"). The strided calls read q, k, v straight out of that map's
[B, T, 3C] output and write O into a [B, T, C] buffer. These tests place the
seeded [B, H, T, D] inputs into such buffers (with padding columns holding
NaN on the input side and a sentinel on the output side), run the strided
path, and check it against the fp64 oracle at the usual bars and against the
contiguous path: the kernels do the same arithmetic whatever the layout, so
O, LSE, dK and dV must agree bit for bit (dQ is summed with atomics in the
bf16 path, so its last bits may differ).
"""
from __future__ import annotations

import pytest
import torch

import causal_self_attention_amd as gattn
from causal_self_attention_amd.inputs import WORKLOADS, make_inputs, workload_inputs
from tests.gpu_helpers import announce, assert_parity, errors, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SENTINEL = 1024.0  # exact in bf16 and fp32
PAD = 64           # padding columns after each row of every buffer


def run_fused(inp: dict, keep_o_lo: bool = True, pad: int = PAD):
    """Forward + backward with q, k, v in a [B, T, 3C + pad] buffer, dO in
    [B, T, C + pad], O into [B, T, C + pad] and fp32 dQ, dK, dV into
    [B, T, 3C + pad]. Returns contiguous CPU results and the buffers."""
    B, H, T, D = inp["q"].shape
    C = H * D
    dt = inp["q"].dtype
    qkv_buf = torch.full((B, T, 3 * C + pad), float("nan"), dtype=dt, device=DEV)
    q, k, v = gattn.split_qkv_heads(qkv_buf[:, :, :3 * C], H)
    for view, name in ((q, "q"), (k, "k"), (v, "v")):
        view.copy_(inp[name].to(DEV))
    do_buf = torch.full((B, T, C + pad), float("nan"), dtype=dt, device=DEV)
    do = gattn.merged_heads_view(do_buf[:, :, :C], H)
    do.copy_(inp["do"].to(DEV))
    y_buf = torch.full((B, T, C + pad), SENTINEL, dtype=dt, device=DEV)
    o_view = gattn.merged_heads_view(y_buf[:, :, :C], H)
    g_buf = torch.full((B, T, 3 * C + pad), SENTINEL, dtype=torch.float32, device=DEV)
    dq, dk, dv = gattn.split_qkv_heads(g_buf[:, :, :3 * C], H)

    o, lse, o_lo = gattn.attention_forward(q, k, v, keep_o_lo=keep_o_lo, out=o_view)
    assert o is o_view
    gattn.attention_backward(q, k, v, o, do, lse, o_lo, grads=(dq, dk, dv))
    torch.cuda.synchronize()
    res = {"o": o.contiguous().cpu(), "lse": lse.cpu(), "dq": dq.contiguous().cpu(),
           "dk": dk.contiguous().cpu(), "dv": dv.contiguous().cpu()}
    return res, {"y": y_buf.cpu(), "g": g_buf.cpu(), "C": C}


def _check_pads(bufs):
    C = bufs["C"]
    assert bool((bufs["y"][:, :, C:].float() == SENTINEL).all()), "O padding overwritten"
    assert bool((bufs["g"][:, :, 3 * C:] == SENTINEL).all()), "gradient padding overwritten"


def _compare_with_contiguous(fused: dict, contig: dict, dtype: str, label: str):
    for name in ("o", "lse", "dk", "dv"):
        assert torch.equal(fused[name], contig[name]), f"{label}: {name} differs from contiguous"
    d = (fused["dq"].double() - contig["dq"].double()).abs().max().item()
    if dtype == "f32":
        assert d == 0.0, f"{label}: fp32 dq differs from contiguous by {d}"
    else:
        assert d <= 1e-5, f"{label}: dq differs from contiguous by {d}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,T", [(2, 3, 333), (1, 2, 129), (2, 1, 1), (1, 4, 64),
                                   (3, 2, 257)])
def test_fused_layout_parity(dtype, B, H, T):
    announce(f"fused layout dtype={dtype} B={B} H={H} T={T}")
    inp = make_inputs(B, H, T, 64, dtype, seed=100 + T)
    fused, bufs = run_fused(inp)
    _check_pads(bufs)
    assert_parity(errors(fused, run_oracle(inp)), dtype, f"fused {dtype} B={B} H={H} T={T}")
    _compare_with_contiguous(fused, run_gpu(inp, o_lo=dtype != "f32"), dtype,
                             f"{dtype} B={B} H={H} T={T}")


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 32), ("f16", 32), ("f32", 32),
                                     ("bf16", 128), ("f16", 128), ("f32", 128)])
def test_fused_layout_other_dtypes_and_head_sizes(dtype, D):
    B, H, T = 2, 3, 200
    announce(f"fused layout dtype={dtype} D={D} B={B} H={H} T={T}")
    inp = make_inputs(B, H, T, D, dtype, seed=300 + D)
    fused, bufs = run_fused(inp)
    _check_pads(bufs)
    assert_parity(errors(fused, run_oracle(inp)), dtype, f"fused {dtype} D={D}")
    _compare_with_contiguous(fused, run_gpu(inp, o_lo=dtype != "f32"), dtype, f"{dtype} D={D}")


def test_fused_layout_without_o_lo():
    announce("fused layout bf16 no o_lo B=2 H=3 T=200")
    inp = make_inputs(2, 3, 200, 64, "bf16", seed=17)
    fused, bufs = run_fused(inp, keep_o_lo=False)
    _check_pads(bufs)
    assert_parity(errors(fused, run_oracle(inp)), "bf16", "fused no o_lo")
    _compare_with_contiguous(fused, run_gpu(inp), "bf16", "no o_lo")


def test_fused_layout_full_size_gpt2_124m():
    """The benchmarked GPT-2 124M attention layer (B=12, H=12, T=1024) in the
    projection layout: oracle on sampled heads, contiguous path on all."""
    w = WORKLOADS["gpt2_124m_bf16_b12_h12_t1024"]
    announce(f"fused layout full size {w.name}")
    inp = workload_inputs(w, seed=0)
    fused, bufs = run_fused(inp)
    _check_pads(bufs)
    heads = [0, 57, 100, w.B * w.H - 1]
    assert_parity(errors(fused, run_oracle(inp, heads), heads), "bf16", f"fused {w.name}")
    _compare_with_contiguous(fused, run_gpu(inp, o_lo=True), "bf16", w.name)


def test_shared_key_value_head_broadcast():
    """Inputs may overlap: one K/V head read by every query head (head stride
    0). Matches the oracle on K, V expanded to every head."""
    B, H, T, D = 2, 4, 190, 64
    announce(f"broadcast K/V head B={B} H={H} T={T}")
    inp = make_inputs(B, H, T, D, "bf16", seed=23)
    k1 = inp["k"][:, :1].contiguous()
    v1 = inp["v"][:, :1].contiguous()
    ref_inp = dict(inp, k=k1.expand(B, H, T, D).contiguous(), v=v1.expand(B, H, T, D).contiguous())
    q = inp["q"].to(DEV)
    do = inp["do"].to(DEV)
    k = k1.to(DEV).expand(B, H, T, D)
    v = v1.to(DEV).expand(B, H, T, D)
    assert k.stride(1) == 0
    o, lse, o_lo = gattn.attention_forward(q, k, v)
    # The backward's dK, dV are per query head (the caller sums them over
    # heads for a shared K, V); compare per head with the expanded oracle.
    dq, dk, dv = gattn.attention_backward(q, k, v, o, do, lse, o_lo)
    torch.cuda.synchronize()
    gpu = {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
    assert_parity(errors(gpu, run_oracle(ref_inp)), "bf16", "broadcast K/V")


def test_padded_head_major_layout():
    """Head-major buffers with padded rows and padded heads (row stride 72 and
    T + 3 rows per head): a layout other than the projection's."""
    B, H, T, D = 2, 3, 150, 64
    announce(f"padded head-major B={B} H={H} T={T}")
    inp = make_inputs(B, H, T, D, "bf16", seed=29)

    def padded(x, fill, dtype):
        buf = torch.full((B, H, T + 3, D + 8), fill, dtype=dtype, device=DEV)
        view = buf[:, :, :T, :D]
        if x is not None:
            view.copy_(x.to(DEV))
        return buf, view

    _, q = padded(inp["q"], float("nan"), torch.bfloat16)
    _, k = padded(inp["k"], float("nan"), torch.bfloat16)
    _, v = padded(inp["v"], float("nan"), torch.bfloat16)
    _, do = padded(inp["do"], float("nan"), torch.bfloat16)
    obuf, o = padded(None, SENTINEL, torch.bfloat16)
    gbufs = [padded(None, SENTINEL, torch.float32) for _ in range(3)]
    assert q.stride() == (H * (T + 3) * 72, (T + 3) * 72, 72, 1)
    _, lse, o_lo = gattn.attention_forward(q, k, v, out=o)
    gattn.attention_backward(q, k, v, o, do, lse, o_lo, grads=tuple(g[1] for g in gbufs))
    torch.cuda.synchronize()
    gpu = {"o": o.contiguous().cpu(), "lse": lse.cpu()}
    for name, (_, view) in zip(("dq", "dk", "dv"), gbufs):
        gpu[name] = view.contiguous().cpu()
    assert_parity(errors(gpu, run_oracle(inp)), "bf16", "padded head-major")
    mask = torch.ones(B, H, T + 3, D + 8, dtype=torch.bool)
    mask[:, :, :T, :D] = False
    assert bool((obuf.cpu().float()[mask] == SENTINEL).all())
    for gbuf, _ in gbufs:
        assert bool((gbuf.cpu()[mask] == SENTINEL).all())


def test_split_phases_equal_one_call():
    """gpt_attn_bwd_prep_strided + gpt_attn_bwd_main_strided give exactly
    what gpt_attn_bwd_strided gives (dQ to atomics rounding)."""
    B, H, T = 2, 2, 300
    announce(f"split strided phases B={B} H={H} T={T}")
    inp = make_inputs(B, H, T, 64, "bf16", seed=31)
    C = H * 64
    qkv = torch.empty(B, T, 3 * C, dtype=torch.bfloat16, device=DEV)
    q, k, v = gattn.split_qkv_heads(qkv, H)
    for view, name in ((q, "q"), (k, "k"), (v, "v")):
        view.copy_(inp[name].to(DEV))
    do = inp["do"].to(DEV)
    o, lse, o_lo = gattn.attention_forward(q, k, v)
    outs = []
    for split in (False, True):
        g = torch.empty(B, T, 3 * C, dtype=torch.float32, device=DEV)
        dq, dk, dv = gattn.split_qkv_heads(g, H)
        ws = torch.empty(gattn.gpt_attn_bwd_workspace_bytes(B, H, T, 64) // 4, dtype=torch.float32,
                         device=DEV)
        if split:
            gattn.gpt_attn_bwd_prep_strided(q, o, o_lo, do, dq, ws)
            gattn.gpt_attn_bwd_main_strided(q, k, v, do, lse, dq, dk, dv, ws)
        else:
            gattn.gpt_attn_bwd_strided(q, k, v, o, o_lo, do, lse, dq, dk, dv, ws)
        torch.cuda.synchronize()
        outs.append(g.cpu())
    C3 = 3 * C
    assert torch.equal(outs[0][:, :, C:C3], outs[1][:, :, C:C3])  # dK, dV
    assert (outs[0][:, :, :C] - outs[1][:, :, :C]).abs().max().item() <= 1e-5


def test_binding_rejects_bad_views():
    inp = make_inputs(1, 2, 16, 64, "bf16", seed=1)
    q = inp["q"].to(DEV)
    q_t = torch.empty(1, 2, 64, 16, dtype=torch.bfloat16, device=DEV).transpose(2, 3)
    assert q_t.shape == q.shape and q_t.stride(3) != 1
    with pytest.raises(ValueError):  # D not contiguous
        gattn.attention_forward(q_t, q, q)
    o_bad = torch.empty(1, 2, 64, dtype=torch.bfloat16, device=DEV).unsqueeze(2).expand(1, 2, 16, 64)
    with pytest.raises(gattn.GptAttnError) as e:  # rows of O overlap
        gattn.attention_forward(q, q, q, out=o_bad)
    assert e.value.status == 6
    torch.cuda.synchronize()
