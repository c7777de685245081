"""Host-side checks of the C ABI, no GPU needed: the library loads, exports
every entry point include/gpt_attn.h declares, and rejects bad arguments
with the documented status before any device work (fake, never-dereferenced
pointer values are used, so a call that got past validation would fail)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import causal_self_attention_amd as gattn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gpt_attn.h")

OK, E_INVAL, E_UNSUP, E_ALIGN, E_WS, E_HIP, E_LAYOUT = 0, 1, 2, 3, 4, 5, 6
DROP = gattn.GptAttnDropout
F32, BF16, F16 = 0, 1, 2
P = 0x10000  # 16-byte aligned fake device address, never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gattn.library_path()):
        from causal_self_attention_amd import build
        build.build()
    return gattn.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt_attn_\w+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    assert declared_functions() == sorted(gattn.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", gattn.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_abi_version_matches_header(lib):
    m = re.search(r"#define GPT_ATTN_ABI_VERSION (\d+)", open(HEADER).read())
    assert gattn.gpt_attn_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for st in range(8):
        assert gattn.gpt_attn_status_string(st)
    assert gattn.gpt_attn_status_string(99) == "unknown status"


def fwd(lib, dtype=BF16, B=1, H=1, T=8, D=64, q=P, k=P, v=P, o=P, lse=P):
    return lib.gpt_attn_fwd(dtype, B, H, T, D, q, k, v, o, lse, None)


def fwd_lo(lib, dtype=BF16, B=1, H=1, T=8, D=64, o_lo=P):
    """The strided forward with contiguous layouts and an o_lo."""
    return lib.gpt_attn_fwd_strided(dtype, B, H, T, D, P, None, P, None, P, None, P, None, o_lo,
                                    None, P, None, None)


def bwd(lib, dtype=BF16, B=1, H=1, T=8, D=64, ptrs=None, ws=P, ws_bytes=1 << 20):
    p = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P)
    p.update(ptrs or {})
    return lib.gpt_attn_bwd(dtype, B, H, T, D, p["q"], p["k"], p["v"], p["o"], p["do"],
                            p["lse"], p["dq"], p["dk"], p["dv"], ws, ws_bytes, None)


def bwd_lo(lib, dtype=BF16, o_lo=P, ws_bytes=1 << 20):
    """The strided backward with contiguous layouts and an o_lo."""
    return lib.gpt_attn_bwd_strided(dtype, 1, 1, 8, 64, P, None, P, None, P, None, P, None, o_lo,
                                    None, P, None, P, P, None, P, None, P, None, P, ws_bytes,
                                    None, None)


def test_forward_validation(lib):
    assert fwd(lib, dtype=3) == E_INVAL
    assert fwd(lib, dtype=-1) == E_INVAL
    assert fwd(lib, B=-1) == E_INVAL
    assert fwd(lib, H=-1) == E_INVAL
    assert fwd(lib, T=-1) == E_INVAL
    assert fwd(lib, D=0) == E_INVAL
    for D in (1, 16, 48, 63, 65, 96, 127, 129, 256):
        assert fwd(lib, D=D) == E_UNSUP
    for name in ("q", "k", "v", "o", "lse"):
        assert fwd(lib, **{name: None}) == E_INVAL, name
        assert fwd(lib, **{name: P + 8}) == E_ALIGN, name
    # o_lo (strided calls) is for the 16-bit dtypes only and must be aligned.
    assert fwd_lo(lib, dtype=F32) == E_INVAL
    assert fwd_lo(lib, o_lo=P + 2) == E_ALIGN
    # B*H*T must stay below 2^31.
    assert fwd(lib, B=1 << 16, H=1 << 15, T=1) == E_INVAL
    assert fwd(lib, B=1 << 10, H=1 << 10, T=1 << 11) == E_INVAL


def test_empty_calls_are_noops(lib):
    for shape in [(0, 1, 8), (1, 0, 8), (1, 1, 0)]:
        B, H, T = shape
        assert fwd(lib, B=B, H=H, T=T, q=None, k=None, v=None, o=None, lse=None) == OK
        assert bwd(lib, B=B, H=H, T=T, ptrs={n: None for n in
                                                ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")},
                   ws=None, ws_bytes=0) == OK
        assert fwd_lo(lib, dtype=F32, B=B, H=H, T=T) == OK
        assert lib.gpt_attn_bwd_workspace_bytes(B, H, T, 64) == 0


def test_backward_validation(lib):
    assert bwd(lib, dtype=-1) == E_INVAL
    assert bwd(lib, D=256) == E_UNSUP
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert bwd(lib, ptrs={name: None}) == E_INVAL, name
        assert bwd(lib, ptrs={name: P + 4}) == E_ALIGN, name
    assert bwd_lo(lib, dtype=F32) == E_INVAL
    assert bwd_lo(lib, o_lo=P + 2) == E_ALIGN
    need = lib.gpt_attn_bwd_workspace_bytes(1, 1, 8, 64)
    assert need == 8 * 4 + 32  # delta, then one chunk's maxima at the next 16-byte boundary
    assert bwd_lo(lib, ws_bytes=need - 1) == E_WS
    assert bwd(lib, ws=None) == E_WS
    assert bwd(lib, ws_bytes=need - 1) == E_WS
    assert bwd(lib, ws=P + 4, ws_bytes=need) == E_ALIGN


def test_workspace_bytes(lib):
    # delta (4 bytes per row), padded to 16 bytes, then 32 bytes per
    # (head, 128-row chunk); the same for every head dimension.
    assert lib.gpt_attn_bwd_workspace_bytes(12, 12, 1024, 64) == 144 * 1024 * 4 + 144 * 8 * 32
    assert lib.gpt_attn_bwd_workspace_bytes(1, 6, 256, 64) == 6 * 256 * 4 + 6 * 2 * 32
    assert lib.gpt_attn_bwd_workspace_bytes(1, 6, 256, 128) == 6 * 256 * 4 + 6 * 2 * 32
    assert lib.gpt_attn_bwd_workspace_bytes(1, 1, 8, 256) == 0
    assert lib.gpt_attn_bwd_workspace_bytes(1, 3, 129, 32) == 1552 + 3 * 2 * 32
    assert lib.gpt_attn_bwd_workspace_bytes(-1, 1, 8, 64) == 0
    assert lib.gpt_attn_bwd_workspace_bytes(1, 1, 0, 64) == 0


def test_binding_refuses_host_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gattn.gpt_attn_fwd(q, q, q, q, torch.zeros(1, 1, 4))


# ---- strided entry points --------------------------------------------------------

L = gattn.GptAttnLayout


def lay(batch, head, row):
    return ctypes.byref(L(batch, head, row))


def fused(B, H, T, D=64):
    """Layouts of q/k/v inside a [B, T, 3C] projection output and of O in [B, T, C]."""
    C = H * D
    return L(3 * T * C, D, 3 * C), L(T * C, D, C)


def fwd_s(lib, dtype=BF16, B=2, H=3, T=8, D=64, lq=None, lk=None, lv=None, lo=None, llo=None,
          o_lo=None, drop=None):
    r = lambda x: None if x is None else ctypes.byref(x)
    return lib.gpt_attn_fwd_strided(dtype, B, H, T, D, P, r(lq), P, r(lk), P, r(lv), P, r(lo),
                                    o_lo, r(llo), P, r(drop), None)


def bwd_s(lib, dtype=BF16, B=2, H=3, T=8, D=64, ws=None, ws_bytes=0, drop=None, **lays):
    r = lambda n: None if lays.get(n) is None else ctypes.byref(lays[n])
    return lib.gpt_attn_bwd_strided(dtype, B, H, T, D, P, r("q"), P, r("k"), P, r("v"), P,
                                    r("o"), None, None, P, r("do"), P, P, r("dq"), P, r("dk"),
                                    P, r("dv"), ws, ws_bytes,
                                    None if drop is None else ctypes.byref(drop), None)


def test_strided_layout_rules_forward(lib):
    B, H, T = 2, 3, 8
    qkv, out = fused(B, H, T)
    # Negative and misaligned strides, for inputs and outputs alike.
    for name in ("lq", "lk", "lv", "lo"):
        assert fwd_s(lib, **{name: L(-8, 64, 64 * H)}) == E_LAYOUT, name
        assert fwd_s(lib, **{name: L(qkv.batch, qkv.head, qkv.row + 1)}) == E_LAYOUT, name
        assert fwd_s(lib, **{name: L(qkv.batch, 60, qkv.row)}) == E_LAYOUT, name
    # fp32 rows are 16-byte aligned at multiples of 4 elements, bf16 at 8.
    assert fwd_s(lib, lq=L(qkv.batch, qkv.head, qkv.row + 4)) == E_LAYOUT
    assert bwd_s(lib, dtype=F32, q=L(4 * 1000, 4 * 100, 68)) == E_WS  # accepted
    assert bwd_s(lib, dtype=F32, q=L(4 * 1000, 4 * 100, 66)) == E_LAYOUT
    assert bwd_s(lib, q=L(4 * 1000, 4 * 100, 68)) == E_LAYOUT  # bf16 needs 8
    # Strides of extent-1 dimensions need no alignment.
    assert bwd_s(lib, B=1, q=L(3, 64, 64 * 3)) == E_WS
    # An output overlapping itself: rows closer than D, heads sharing rows,
    # batches sharing heads.
    assert fwd_s(lib, lo=L(out.batch, out.head, 32)) == E_LAYOUT
    assert fwd_s(lib, lo=L(out.batch, 0, out.row)) == E_LAYOUT
    assert fwd_s(lib, lo=L(0, out.head, out.row)) == E_LAYOUT
    assert fwd_s(lib, o_lo=P, llo=L(out.batch, out.head, 8)) == E_LAYOUT
    assert fwd_s(lib, dtype=F32, lo=L(out.batch, out.head, 60)) == E_LAYOUT
    # Offsets inside one head must fit 32 bits.
    assert fwd_s(lib, T=1 << 16, lq=L(0, 64, 1 << 16)) == E_LAYOUT


def test_strided_backward_accepts_the_fused_layout(lib):
    """Every layout check passes for the projection layout (the call then
    stops at the missing workspace, before any launch)."""
    B, H, T = 2, 3, 8
    qkv, out = fused(B, H, T)
    g = L(3 * T * H * 64, 64, 3 * H * 64)  # fp32 gradients in a [B, T, 3C] buffer
    kw = dict(q=qkv, k=qkv, v=qkv, o=out, do=out, dq=g, dk=g, dv=g)
    assert bwd_s(lib, **kw) == E_WS
    assert bwd_s(lib, dtype=F32, **kw) == E_WS
    # Inputs may overlap (a broadcast head), outputs may not.
    assert bwd_s(lib, **{**kw, "k": L(3 * T * H * 64, 0, 3 * H * 64)}) == E_WS
    assert bwd_s(lib, **{**kw, "dk": L(3 * T * H * 64, 0, 3 * H * 64)}) == E_LAYOUT
    assert bwd_s(lib, **{**kw, "dq": L(-4, 64, 64)}) == E_LAYOUT
    assert bwd_s(lib, **{**kw, "do": L(8, 64, 3)}) == E_LAYOUT


def test_plain_calls_equal_strided_calls_with_null_layouts(lib):
    # Same validation outcome either way.
    assert fwd_s(lib, D=256) == fwd(lib, D=256) == E_UNSUP
    assert bwd_s(lib) == E_WS
    assert lib.gpt_attn_bwd_prep_strided(BF16, 1, 1, 8, 64, P, None, P, None, None, None, P, None,
                                         P, ctypes.byref(L(0, 0, 32)), P, 1 << 20,
                                         None) == E_LAYOUT
    # The 16-bit prep phase reads q (for its maxima); fp32 does not need it.
    assert lib.gpt_attn_bwd_prep(BF16, 1, 1, 8, 64, None, P, P, P, P, 1 << 20, None) == E_INVAL
    assert lib.gpt_attn_bwd_prep(BF16, 1, 1, 8, 64, P + 2, P, P, P, P, 1 << 20, None) == E_ALIGN
    assert lib.gpt_attn_bwd_main_strided(BF16, 1, 1, 8, 64, P, None, P, None, P, None, P, None,
                                         P, P, None, P, None, P, ctypes.byref(L(0, 0, 32)), None,
                                         0, None, None) == E_LAYOUT


def test_view_helpers_match_the_fused_layout():
    import torch
    B, T, H, D = 2, 5, 3, 64
    qkv = torch.arange(B * T * 3 * H * D, dtype=torch.float32).view(B, T, 3 * H * D)
    q, k, v = gattn.split_qkv_heads(qkv, H)
    qkv_l, out_l = fused(B, H, T)
    for i, t in enumerate((q, k, v)):
        assert tuple(t.shape) == (B, H, T, D)
        assert t.stride() == (qkv_l.batch, qkv_l.head, qkv_l.row, 1)
        assert t.storage_offset() == i * H * D
        # element (b, h, t, d) is the projection's column (i*C + h*D + d) of token t
        assert t[1, 2, 3, 4].item() == qkv[1, 3, i * H * D + 2 * D + 4].item()
    y = torch.zeros(B, T, H * D)
    o = gattn.merged_heads_view(y, H)
    assert o.stride() == (out_l.batch, out_l.head, out_l.row, 1)
    o[1, 2, 3, 4] = 7.0
    assert y[1, 3, 2 * D + 4].item() == 7.0


# ---- dropout descriptor ------------------------------------------------------------

def test_dropout_descriptor_validation(lib):
    """Bad probabilities are rejected before any launch; good descriptors pass
    validation (the backward then stops at the missing workspace)."""
    for p in (-0.1, 1.0, 1.5, 0.999995, float("nan"), float("inf")):
        assert fwd_s(lib, drop=DROP(p, 1, 0)) == E_INVAL, p
        assert bwd_s(lib, drop=DROP(p, 1, 0)) == E_INVAL, p
        assert bwd_s(lib, dtype=F32, drop=DROP(p, 1, 0)) == E_INVAL, p
    for p in (0.0, 0.1, 0.2, 0.99999):
        assert bwd_s(lib, drop=DROP(p, 2**64 - 1, 2**32 - 1)) == E_WS, p
    # Shape errors still come first.
    assert fwd_s(lib, D=256, drop=DROP(2.0, 0, 0)) == E_UNSUP


def test_dropout_mask_entry_validation(lib):
    d = ctypes.byref(DROP(0.2, 5, 1))
    assert lib.gpt_attn_dropout_mask(1, 1, 8, None, P, None) == E_INVAL
    assert lib.gpt_attn_dropout_mask(-1, 1, 8, d, P, None) == E_INVAL
    assert lib.gpt_attn_dropout_mask(1, 1, 8, ctypes.byref(DROP(1.0, 5, 1)), P, None) == E_INVAL
    assert lib.gpt_attn_dropout_mask(1, 1, 8, d, None, None) == E_INVAL
    assert lib.gpt_attn_dropout_mask(1 << 12, 1 << 10, 1 << 10, d, P, None) == E_INVAL  # 2^42 B
    assert lib.gpt_attn_dropout_mask(0, 1, 8, d, None, None) == OK   # empty: nothing to do
    assert lib.gpt_attn_dropout_mask(1, 1, 0, d, None, None) == OK


# ---- decode ----------------------------------------------------------------------------

def dec(lib, dtype=BF16, B=2, H=3, L=100, D=64, q=P, k=P, v=P, lengths=None, o=P, lse=P,
        ws=None, ws_bytes=0, lk=None, lo=None):
    r = lambda x: None if x is None else ctypes.byref(x)
    return lib.gpt_attn_decode(dtype, B, H, L, D, q, None, k, r(lk), v, None, lengths, o, r(lo),
                               lse, ws, ws_bytes, None)


def test_decode_validation(lib):
    need = lib.gpt_attn_decode_workspace_bytes(BF16, 2, 3, 100, 64)
    assert need == 2 * 3 * 1 * 132 * 4      # one 128-key chunk per head at most
    assert lib.gpt_attn_decode_workspace_bytes(BF16, 64, 12, 1024, 64) == 768 * 8 * 132 * 4
    assert lib.gpt_attn_decode_workspace_bytes(BF16, 2, 3, 0, 64) == 0
    assert lib.gpt_attn_decode_workspace_bytes(BF16, 2, 3, 100, 128) == need
    assert lib.gpt_attn_decode_workspace_bytes(BF16, 2, 3, 100, 256) == 0
    assert lib.gpt_attn_decode_workspace_bytes(F16, 2, 3, 100, 32) == need
    assert dec(lib, D=256) == E_UNSUP
    assert dec(lib, dtype=5) == E_INVAL
    assert dec(lib, L=-1) == E_INVAL
    for name in ("q", "k", "v", "o", "lse"):
        assert dec(lib, **{name: None}) == E_INVAL, name
        assert dec(lib, **{name: P + 4}) == E_ALIGN, name
    assert dec(lib, lengths=P + 4) == E_ALIGN
    assert dec(lib) == E_WS                             # every check passed but the workspace
    assert dec(lib, ws=P, ws_bytes=need - 1) == E_WS
    assert dec(lib, ws=P + 4, ws_bytes=need) == E_ALIGN
    assert dec(lib, lk=L(-8, 64, 64)) == E_LAYOUT
    assert dec(lib, lo=L(64, 0, 64)) == E_LAYOUT       # heads of O overlap
    assert dec(lib, B=0, q=None, k=None, v=None, o=None, lse=None) == OK


def test_sixteen_bit_dtypes_and_head_sizes_share_the_rules(lib):
    """fp16 and D = 32 go through the same validation (every call below stops
    at a validation error, before any launch)."""
    for dt in (BF16, F16):
        for D in (32, 64):
            assert fwd(lib, dtype=dt, D=D, q=None) == E_INVAL
            assert fwd(lib, dtype=dt, D=D, o=P + 2) == E_ALIGN
            assert bwd(lib, dtype=dt, D=D, ws=None) == E_WS
            assert bwd(lib, dtype=dt, D=D, ptrs={"dq": None}) == E_INVAL
    # o_lo is allowed for both 16-bit types, not for fp32.
    assert fwd_lo(lib, dtype=F16, o_lo=P + 2) == E_ALIGN
    assert fwd_lo(lib, dtype=F32, D=32) == E_INVAL
    # fp16 rows are 16-byte aligned at multiples of 8 elements.
    assert bwd_s(lib, dtype=F16, q=L(8 * 300, 8 * 40, 8 * 7)) == E_WS
    assert bwd_s(lib, dtype=F16, q=L(8 * 300, 8 * 40, 60)) == E_LAYOUT


# ---- the allocation-free backward --------------------------------------------------

def test_noalloc_validation_before_any_device_work(lib):
    def call(dtype=BF16, B=1, H=1, T=8, D=64, q=P, dq=P):
        return lib.gpt_attn_bwd_noalloc(dtype, B, H, T, D, q, P, P, P, P, P, dq, P, P, None)
    assert call(D=256) == E_UNSUP
    assert call(q=None) == E_INVAL
    assert call(dq=P + 4) == E_ALIGN
    # 64 * 64 * 1024 rows need 16.8 MB of workspace, beyond the 8 MiB scratch.
    assert lib.gpt_attn_bwd_workspace_bytes(64, 64, 1024, 64) > gattn.NOALLOC_SCRATCH_BYTES
    assert call(B=64, H=64, T=1024) == 7
    assert call(B=0) == OK
    text = open(HEADER).read()
    assert f"#define GPT_ATTN_NOALLOC_SCRATCH_BYTES (8u << 20)" in text
    assert gattn.NOALLOC_SCRATCH_BYTES == 8 << 20
    assert "static" in gattn.gpt_attn_status_string(7)
