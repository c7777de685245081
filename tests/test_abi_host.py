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

OK, E_INVAL, E_UNSUP, E_ALIGN, E_WS, E_HIP = 0, 1, 2, 3, 4, 5
F32, BF16 = 0, 1
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
    for st in range(6):
        assert gattn.gpt_attn_status_string(st)
    assert gattn.gpt_attn_status_string(99) == "unknown status"


def fwd(lib, dtype=BF16, B=1, H=1, T=8, D=64, q=P, k=P, v=P, o=P, o_lo=None, lse=P):
    return lib.gpt_attn_fwd(dtype, B, H, T, D, q, k, v, o, o_lo, lse, None)


def bwd(lib, dtype=BF16, B=1, H=1, T=8, D=64, ptrs=None, ws=P, ws_bytes=1 << 20):
    p = dict(q=P, k=P, v=P, o=P, o_lo=None, do=P, lse=P, dq=P, dk=P, dv=P)
    p.update(ptrs or {})
    return lib.gpt_attn_bwd(dtype, B, H, T, D, p["q"], p["k"], p["v"], p["o"], p["o_lo"],
                            p["do"], p["lse"], p["dq"], p["dk"], p["dv"], ws, ws_bytes, None)


def test_forward_validation(lib):
    assert fwd(lib, dtype=2) == E_INVAL
    assert fwd(lib, B=-1) == E_INVAL
    assert fwd(lib, H=-1) == E_INVAL
    assert fwd(lib, T=-1) == E_INVAL
    assert fwd(lib, D=0) == E_INVAL
    for D in (1, 32, 63, 65, 128):
        assert fwd(lib, D=D) == E_UNSUP
    for name in ("q", "k", "v", "o", "lse"):
        assert fwd(lib, **{name: None}) == E_INVAL, name
        assert fwd(lib, **{name: P + 8}) == E_ALIGN, name
    # o_lo is bf16-only and must be aligned.
    assert fwd(lib, dtype=F32, o_lo=P) == E_INVAL
    assert fwd(lib, o_lo=P + 2) == E_ALIGN
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
        assert fwd(lib, dtype=F32, B=B, H=H, T=T, o_lo=P) == OK
        assert lib.gpt_attn_bwd_workspace_bytes(BF16, B, H, T, 64) == 0


def test_backward_validation(lib):
    assert bwd(lib, dtype=-1) == E_INVAL
    assert bwd(lib, D=32) == E_UNSUP
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert bwd(lib, ptrs={name: None}) == E_INVAL, name
        assert bwd(lib, ptrs={name: P + 4}) == E_ALIGN, name
    assert bwd(lib, dtype=F32, ptrs={"o_lo": P}) == E_INVAL
    assert bwd(lib, ptrs={"o_lo": P + 2}) == E_ALIGN
    need = lib.gpt_attn_bwd_workspace_bytes(BF16, 1, 1, 8, 64)
    assert need == 8 * 4
    assert bwd(lib, ws=None) == E_WS
    assert bwd(lib, ws_bytes=need - 1) == E_WS
    assert bwd(lib, ws=P + 4, ws_bytes=need) == E_ALIGN


def test_workspace_bytes(lib):
    assert lib.gpt_attn_bwd_workspace_bytes(BF16, 12, 12, 1024, 64) == 12 * 12 * 1024 * 4
    assert lib.gpt_attn_bwd_workspace_bytes(F32, 1, 6, 256, 64) == 6 * 256 * 4
    assert lib.gpt_attn_bwd_workspace_bytes(BF16, 1, 1, 8, 32) == 0
    assert lib.gpt_attn_bwd_workspace_bytes(7, 1, 1, 8, 64) == 0
    assert lib.gpt_attn_bwd_workspace_bytes(BF16, -1, 1, 8, 64) == 0


def test_binding_refuses_host_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gattn.gpt_attn_fwd(q, q, q, q, None, torch.zeros(1, 1, 4))
