"""Fused causal self-attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/gpt_attn.h`` (library
``libgptattn.so``, built in-tree by ``python -m causal_self_attention_amd.build``).
The functions here only marshal torch CUDA tensors into pointers, sizes and
the current HIP stream; every step of the computation runs in the library's
HIP kernels. If the library is missing or cannot be loaded, every call raises
``RuntimeError``: there is no fallback.

The names mirror the C entry points:

  gpt_attn_fwd(q, k, v, o, o_lo, lse)                -> None (writes o, o_lo, lse)
  gpt_attn_bwd(q, k, v, o, o_lo, dout, lse, dq, dk, dv, workspace) -> None
  gpt_attn_bwd_prep(o, o_lo, dout, dq, workspace)     -> None (phase 1 of bwd)
  gpt_attn_bwd_main(q, k, v, dout, lse, dq, dk, dv, workspace) -> None (phase 2)
  gpt_attn_bwd_workspace_bytes(dtype, B, H, T, D)    -> int
  gpt_attn_status_string(status)                     -> str
  gpt_attn_abi_version()                             -> int

plus two allocating conveniences, ``attention_forward`` and
``attention_backward``. Tensors are [B, H, T, D] contiguous; q, k, v, o, dout
are float32 or bfloat16; lse [B, H, T] and dq, dk, dv are float32. o_lo
(bf16 only, may be None) is the bf16 low part of the forward's fp32 O, which
the backward uses for an accurate delta = rowsum(dO * O).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "GptAttnError", "library_path", "load_library", "gpt_attn_fwd", "gpt_attn_bwd",
    "gpt_attn_bwd_prep", "gpt_attn_bwd_main", "gpt_attn_bwd_workspace_bytes",
    "gpt_attn_status_string", "gpt_attn_abi_version", "attention_forward", "attention_backward", "DTYPE_CODES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgptattn.so"
_lib = None

GPT_ATTN_F32 = 0
GPT_ATTN_BF16 = 1
DTYPE_CODES = {"f32": GPT_ATTN_F32, "bf16": GPT_ATTN_BF16}

#: every symbol include/gpt_attn.h declares
EXPORTED_SYMBOLS = ("gpt_attn_fwd", "gpt_attn_bwd", "gpt_attn_bwd_prep", "gpt_attn_bwd_main",
                    "gpt_attn_bwd_workspace_bytes", "gpt_attn_status_string",
                    "gpt_attn_abi_version")


class GptAttnError(RuntimeError):
    def __init__(self, entry: str, status: int):
        self.status = status
        super().__init__(f"{entry} failed: status {status} ({gpt_attn_status_string(status)})")


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load libgptattn.so (once). Raises RuntimeError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m causal_self_attention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.gpt_attn_fwd.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp]
    lib.gpt_attn_fwd.restype = i
    lib.gpt_attn_bwd.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                 vp]
    lib.gpt_attn_bwd.restype = i
    lib.gpt_attn_bwd_prep.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, sz, vp]
    lib.gpt_attn_bwd_prep.restype = i
    lib.gpt_attn_bwd_main.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gpt_attn_bwd_main.restype = i
    lib.gpt_attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.gpt_attn_bwd_workspace_bytes.restype = sz
    lib.gpt_attn_status_string.argtypes = [i]
    lib.gpt_attn_status_string.restype = ctypes.c_char_p
    lib.gpt_attn_abi_version.argtypes = []
    lib.gpt_attn_abi_version.restype = i
    _lib = lib
    return lib


def gpt_attn_status_string(status: int) -> str:
    return load_library().gpt_attn_status_string(int(status)).decode()


def gpt_attn_abi_version() -> int:
    return int(load_library().gpt_attn_abi_version())


def gpt_attn_bwd_workspace_bytes(dtype: int | str, B: int, H: int, T: int, D: int) -> int:
    code = DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    return int(load_library().gpt_attn_bwd_workspace_bytes(code, B, H, T, D))


# ---- marshalling helpers ------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return GPT_ATTN_F32
    if t.dtype == torch.bfloat16:
        return GPT_ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a CUDA (HIP) device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _stream(device, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _bhtd(q):
    if q.dim() != 4:
        raise ValueError(f"expected [B, H, T, D], got shape {tuple(q.shape)}")
    return tuple(int(x) for x in q.shape)


def gpt_attn_fwd(q, k, v, o, o_lo, lse, stream=None) -> None:
    """Enqueue the forward on ``stream`` (default: torch's current stream)."""
    B, H, T, D = _bhtd(q)
    st = load_library().gpt_attn_fwd(_dtype_code(q), B, H, T, D, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(o), _ptr(o_lo), _ptr(lse), _stream(q.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_fwd", st)


def gpt_attn_bwd(q, k, v, o, o_lo, dout, lse, dq, dk, dv, workspace, stream=None) -> None:
    """Enqueue the backward on ``stream`` (default: torch's current stream)."""
    B, H, T, D = _bhtd(q)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().gpt_attn_bwd(_dtype_code(q), B, H, T, D, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(o), _ptr(o_lo), _ptr(dout), _ptr(lse), _ptr(dq),
                                     _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                                     _stream(q.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_bwd", st)


def _ws_bytes(workspace) -> int:
    return workspace.numel() * workspace.element_size() if workspace is not None else 0


def gpt_attn_bwd_prep(o, o_lo, dout, dq, workspace, stream=None) -> None:
    """Enqueue the backward's preprocess phase (delta, and dq zeroing)."""
    B, H, T, D = _bhtd(o)
    st = load_library().gpt_attn_bwd_prep(_dtype_code(o), B, H, T, D, _ptr(o), _ptr(o_lo),
                                          _ptr(dout), _ptr(dq), _ptr(workspace),
                                          _ws_bytes(workspace), _stream(o.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_bwd_prep", st)


def gpt_attn_bwd_main(q, k, v, dout, lse, dq, dk, dv, workspace, stream=None) -> None:
    """Enqueue the backward's main phase (needs gpt_attn_bwd_prep first)."""
    B, H, T, D = _bhtd(q)
    st = load_library().gpt_attn_bwd_main(_dtype_code(q), B, H, T, D, _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                          _ptr(workspace), _ws_bytes(workspace),
                                          _stream(q.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_bwd_main", st)


def attention_forward(q, k, v, stream=None, keep_o_lo: bool = True):
    """Allocate O (dtype of q), LSE (fp32) and, for bf16 with keep_o_lo, the
    low part o_lo; run the forward; return (o, lse, o_lo) (o_lo may be None)."""
    import torch
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v must share shape and dtype")
    o = torch.empty_like(q)
    o_lo = torch.empty_like(q) if (keep_o_lo and q.dtype == torch.bfloat16) else None
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    gpt_attn_fwd(q, k, v, o, o_lo, lse, stream)
    return o, lse, o_lo


def attention_backward(q, k, v, o, dout, lse, o_lo=None, stream=None, workspace=None):
    """Allocate fp32 dQ, dK, dV (and the workspace unless given), run the
    backward, return (dq, dk, dv)."""
    import torch
    B, H, T, D = _bhtd(q)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    if workspace is None:
        nbytes = gpt_attn_bwd_workspace_bytes(_dtype_code(q), B, H, T, D)
        workspace = torch.empty(max(1, (nbytes + 3) // 4), dtype=torch.float32, device=q.device)
    gpt_attn_bwd(q, k, v, o, o_lo, dout, lse, dq, dk, dv, workspace, stream)
    return dq, dk, dv
