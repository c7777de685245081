"""Fused causal self-attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/gpt_attn.h`` (library
``libgptattn.so``, built in-tree by ``python -m causal_self_attention_amd.build``).
The functions here only marshal torch CUDA tensors into pointers, sizes and
the current HIP stream; every step of the computation runs in the library's
HIP kernels. If the library is missing or cannot be loaded, every call raises
``RuntimeError``: there is no fallback.

The names mirror the C entry points:

  gpt_attn_fwd(q, k, v, o, lse)                      -> None (writes o, lse)
  gpt_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace) -> None
  gpt_attn_bwd_prep(q, o, dout, dq, workspace)        -> None (phase 1 of bwd)
  gpt_attn_bwd_main(q, k, v, dout, lse, dq, dk, dv, workspace) -> None (phase 2)
  gpt_attn_bwd_workspace_bytes(B, H, T, D)           -> int
  gpt_attn_status_string(status)                     -> str
  gpt_attn_abi_version()                             -> int

and the strided forms gpt_attn_fwd_strided, gpt_attn_bwd_strided,
gpt_attn_bwd_prep_strided, gpt_attn_bwd_main_strided (the same arguments
plus the optional o_lo, the low part of the forward's fp32 O; each
tensor's own strides become its gpt_attn_layout; the forward and backward
ones take an optional ``dropout=(p, seed, offset)``), gpt_attn_dropout_mask
(the keep mask the kernels derive, written out), gpt_attn_decode (one query
per head against a key/value cache) with gpt_attn_decode_workspace_bytes,
plus three allocating
conveniences, ``attention_forward``, ``attention_backward`` and
``attention_decode``, and the view
helpers ``split_qkv_heads`` / ``merged_heads_view`` for the fused [B, T, 3C]
projection layout. Tensors are logically [B, H, T, D]: contiguous for the
plain calls, any layout with unit stride along D for the strided ones; q, k,
v, o, dout are float32, bfloat16 or float16 with D in {32, 64, 128}; lse
[B, H, T] (contiguous) and dq, dk, dv are float32. o_lo (16-bit dtypes only,
may be None) is the low part of the forward's fp32 O in the same dtype,
which the backward uses for an accurate delta = rowsum(dO * O).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "GptAttnError", "library_path", "load_library", "gpt_attn_fwd", "gpt_attn_bwd",
    "gpt_attn_bwd_prep", "gpt_attn_bwd_main", "gpt_attn_bwd_workspace_bytes",
    "gpt_attn_status_string", "gpt_attn_abi_version", "gpt_attn_fwd_strided",
    "gpt_attn_bwd_strided", "gpt_attn_bwd_prep_strided", "gpt_attn_bwd_main_strided",
    "attention_forward", "attention_backward", "split_qkv_heads", "merged_heads_view",
    "DTYPE_CODES", "GptAttnLayout", "GptAttnDropout", "gpt_attn_dropout_mask",
    "gpt_attn_decode", "gpt_attn_decode_workspace_bytes", "attention_decode",
    "gpt_attn_bwd_noalloc", "NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgptattn.so"
_lib = None

GPT_ATTN_F32 = 0
GPT_ATTN_BF16 = 1
GPT_ATTN_F16 = 2
DTYPE_CODES = {"f32": GPT_ATTN_F32, "bf16": GPT_ATTN_BF16, "f16": GPT_ATTN_F16}

#: every symbol include/gpt_attn.h declares
EXPORTED_SYMBOLS = ("gpt_attn_fwd", "gpt_attn_bwd", "gpt_attn_bwd_prep", "gpt_attn_bwd_main",
                    "gpt_attn_bwd_noalloc",
                    "gpt_attn_fwd_strided", "gpt_attn_bwd_strided", "gpt_attn_bwd_prep_strided",
                    "gpt_attn_bwd_main_strided", "gpt_attn_dropout_mask", "gpt_attn_decode",
                    "gpt_attn_decode_workspace_bytes", "gpt_attn_bwd_workspace_bytes",
                    "gpt_attn_status_string", "gpt_attn_abi_version")

ABI_VERSION = 7
NOALLOC_SCRATCH_BYTES = 8 << 20


class GptAttnLayout(ctypes.Structure):
    """struct gpt_attn_layout: element strides (batch, head, row) of a
    logically [B, H, T, D] operand whose D elements are contiguous."""
    _fields_ = [("batch", ctypes.c_longlong), ("head", ctypes.c_longlong),
                ("row", ctypes.c_longlong)]


class GptAttnDropout(ctypes.Structure):
    """struct gpt_attn_dropout: drop probability p (0 <= p < 1, rounded to a
    multiple of 2^-16), 64-bit Philox seed and 32-bit stream offset."""
    _fields_ = [("p", ctypes.c_double), ("seed", ctypes.c_ulonglong),
                ("offset", ctypes.c_uint)]


def _dropout_arg(dropout):
    """None, a GptAttnDropout, or (p, seed[, offset]) -> pointer or None."""
    if dropout is None:
        return None
    if not isinstance(dropout, GptAttnDropout):
        p, seed, *rest = dropout
        dropout = GptAttnDropout(float(p), int(seed) & (2**64 - 1),
                                 int(rest[0] if rest else 0) & 0xFFFFFFFF)
    return ctypes.byref(dropout)


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
    lib.gpt_attn_fwd.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, vp]
    lib.gpt_attn_fwd.restype = i
    lib.gpt_attn_bwd.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gpt_attn_bwd.restype = i
    lib.gpt_attn_bwd_prep.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, sz, vp]
    lib.gpt_attn_bwd_prep.restype = i
    lib.gpt_attn_bwd_main.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gpt_attn_bwd_noalloc.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gpt_attn_bwd_noalloc.restype = i
    lib.gpt_attn_bwd_main.restype = i
    lp = ctypes.POINTER(GptAttnLayout)
    dp_ = ctypes.POINTER(GptAttnDropout)
    lib.gpt_attn_fwd_strided.argtypes = [i, i, i, i, i, vp, lp, vp, lp, vp, lp, vp, lp, vp, lp,
                                         vp, dp_, vp]
    lib.gpt_attn_fwd_strided.restype = i
    lib.gpt_attn_bwd_strided.argtypes = [i, i, i, i, i, vp, lp, vp, lp, vp, lp, vp, lp, vp, lp,
                                         vp, lp, vp, vp, lp, vp, lp, vp, lp, vp, sz, dp_, vp]
    lib.gpt_attn_bwd_strided.restype = i
    lib.gpt_attn_bwd_prep_strided.argtypes = [i, i, i, i, i, vp, lp, vp, lp, vp, lp, vp, lp, vp,
                                              lp, vp, sz, vp]
    lib.gpt_attn_bwd_prep_strided.restype = i
    lib.gpt_attn_bwd_main_strided.argtypes = [i, i, i, i, i, vp, lp, vp, lp, vp, lp, vp, lp, vp,
                                              vp, lp, vp, lp, vp, lp, vp, sz, dp_, vp]
    lib.gpt_attn_bwd_main_strided.restype = i
    lib.gpt_attn_dropout_mask.argtypes = [i, i, i, dp_, vp, vp]
    lib.gpt_attn_dropout_mask.restype = i
    lib.gpt_attn_decode.argtypes = [i, i, i, i, i, vp, lp, vp, lp, vp, lp, vp, vp, lp, vp, vp,
                                    sz, vp]
    lib.gpt_attn_decode.restype = i
    lib.gpt_attn_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.gpt_attn_decode_workspace_bytes.restype = sz
    lib.gpt_attn_bwd_workspace_bytes.argtypes = [i, i, i, i]
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


def gpt_attn_bwd_workspace_bytes(B: int, H: int, T: int, D: int) -> int:
    return int(load_library().gpt_attn_bwd_workspace_bytes(B, H, T, D))


# ---- marshalling helpers ------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return GPT_ATTN_F32
    if t.dtype == torch.bfloat16:
        return GPT_ATTN_BF16
    if t.dtype == torch.float16:
        return GPT_ATTN_F16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32, bfloat16 or float16")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a CUDA (HIP) device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _sptr(t):
    """Pointer and gpt_attn_layout of a logically [B, H, T, D] view (unit
    stride along D), or (None, None) for None."""
    if t is None:
        return None, None
    if not t.is_cuda:
        raise ValueError("expected a CUDA (HIP) device tensor")
    if t.dim() != 4:
        raise ValueError(f"expected a [B, H, T, D] view, got shape {tuple(t.shape)}")
    if t.numel() == 0:
        return None, None
    if t.stride(3) != 1:
        raise ValueError("the D dimension must be contiguous (stride 1)")
    lay = GptAttnLayout(t.stride(0), t.stride(1), t.stride(2))
    return ctypes.c_void_p(t.data_ptr()), ctypes.byref(lay)


def _same_shape(ref, *ts):
    for t in ts:
        if t is not None and tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"shape {tuple(t.shape)} differs from {tuple(ref.shape)}")


def _stream(device, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _bhtd(q):
    if q.dim() != 4:
        raise ValueError(f"expected [B, H, T, D], got shape {tuple(q.shape)}")
    return tuple(int(x) for x in q.shape)


def gpt_attn_fwd(q, k, v, o, lse, stream=None) -> None:
    """Enqueue the forward on ``stream`` (default: torch's current stream)."""
    B, H, T, D = _bhtd(q)
    st = load_library().gpt_attn_fwd(_dtype_code(q), B, H, T, D, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(o), _ptr(lse), _stream(q.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_fwd", st)


def gpt_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, stream=None) -> None:
    """Enqueue the backward on ``stream`` (default: torch's current stream)."""
    B, H, T, D = _bhtd(q)
    st = load_library().gpt_attn_bwd(_dtype_code(q), B, H, T, D, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                                     _ptr(dv), _ptr(workspace), _ws_bytes(workspace),
                                     _stream(q.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_bwd", st)


def gpt_attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, stream=None) -> None:
    """gpt_attn_bwd with the library's static per-GPU scratch in place of a
    workspace (allocates nothing; calls on one GPU must not overlap)."""
    B, H, T, D = _bhtd(q)
    st = load_library().gpt_attn_bwd_noalloc(_dtype_code(q), B, H, T, D, _ptr(q), _ptr(k),
                                             _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                             _ptr(dk), _ptr(dv), _stream(q.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_bwd_noalloc", st)


def _ws_bytes(workspace) -> int:
    return workspace.numel() * workspace.element_size() if workspace is not None else 0


def gpt_attn_bwd_prep(q, o, dout, dq, workspace, stream=None) -> None:
    """Enqueue the backward's preprocess phase (delta, per-chunk maxima, and
    dq zeroing)."""
    B, H, T, D = _bhtd(o)
    st = load_library().gpt_attn_bwd_prep(_dtype_code(o), B, H, T, D, _ptr(q), _ptr(o),
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


# ---- strided forms ------------------------------------------------------------

def gpt_attn_fwd_strided(q, k, v, o, o_lo, lse, stream=None, dropout=None) -> None:
    """gpt_attn_fwd on [B, H, T, D] views of any layout with unit D stride;
    ``dropout`` = None or (p, seed, offset)."""
    B, H, T, D = _bhtd(q)
    _same_shape(q, k, v, o, o_lo)
    args = []
    for t in (q, k, v, o, o_lo):
        args.extend(_sptr(t))
    st = load_library().gpt_attn_fwd_strided(_dtype_code(q), B, H, T, D, *args, _ptr(lse),
                                             _dropout_arg(dropout), _stream(q.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_fwd_strided", st)


def gpt_attn_bwd_strided(q, k, v, o, o_lo, dout, lse, dq, dk, dv, workspace,
                         stream=None, dropout=None) -> None:
    """gpt_attn_bwd on [B, H, T, D] views of any layout with unit D stride;
    ``dropout`` must be the forward's."""
    B, H, T, D = _bhtd(q)
    _same_shape(q, k, v, o, o_lo, dout, dq, dk, dv)
    args = []
    for t in (q, k, v, o, o_lo, dout):
        args.extend(_sptr(t))
    args.append(_ptr(lse))
    for t in (dq, dk, dv):
        args.extend(_sptr(t))
    st = load_library().gpt_attn_bwd_strided(_dtype_code(q), B, H, T, D, *args, _ptr(workspace),
                                             _ws_bytes(workspace), _dropout_arg(dropout),
                                             _stream(q.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_bwd_strided", st)


def gpt_attn_bwd_prep_strided(q, o, o_lo, dout, dq, workspace, stream=None) -> None:
    """gpt_attn_bwd_prep on [B, H, T, D] views (unit D stride), with the
    optional o_lo."""
    B, H, T, D = _bhtd(o)
    _same_shape(o, q, o_lo, dout, dq)
    args = []
    for t in (q, o, o_lo, dout, dq):
        args.extend(_sptr(t))
    st = load_library().gpt_attn_bwd_prep_strided(_dtype_code(o), B, H, T, D, *args,
                                                  _ptr(workspace), _ws_bytes(workspace),
                                                  _stream(o.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_bwd_prep_strided", st)


def gpt_attn_bwd_main_strided(q, k, v, dout, lse, dq, dk, dv, workspace, stream=None,
                              dropout=None) -> None:
    """gpt_attn_bwd_main on [B, H, T, D] views (unit D stride)."""
    B, H, T, D = _bhtd(q)
    _same_shape(q, k, v, dout, dq, dk, dv)
    args = []
    for t in (q, k, v, dout):
        args.extend(_sptr(t))
    args.append(_ptr(lse))
    for t in (dq, dk, dv):
        args.extend(_sptr(t))
    st = load_library().gpt_attn_bwd_main_strided(_dtype_code(q), B, H, T, D, *args,
                                                  _ptr(workspace), _ws_bytes(workspace),
                                                  _dropout_arg(dropout),
                                                  _stream(q.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_bwd_main_strided", st)


def gpt_attn_dropout_mask(B: int, H: int, T: int, dropout, mask, stream=None) -> None:
    """Write the keep mask (uint8 [B, H, T, T], contiguous, 1 = visible and
    kept) the attention kernels derive for ``dropout`` = (p, seed, offset)."""
    import torch
    if mask.dtype != torch.uint8 or tuple(mask.shape) != (B, H, T, T):
        raise ValueError("mask must be uint8 of shape [B, H, T, T]")
    st = load_library().gpt_attn_dropout_mask(B, H, T, _dropout_arg(dropout), _ptr(mask),
                                              _stream(mask.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_dropout_mask", st)


# ---- one query against a key/value cache -------------------------------------------

def gpt_attn_decode_workspace_bytes(dtype: int | str, B: int, H: int, L: int, D: int) -> int:
    code = DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    return int(load_library().gpt_attn_decode_workspace_bytes(code, B, H, L, D))


def gpt_attn_decode(q, k_cache, v_cache, lengths, o, lse, workspace, stream=None) -> None:
    """q, o [B, H, D] and caches [B, H, L, D] (any layout with unit D
    stride); lengths: int32 [B] device tensor or None (L everywhere); lse
    [B, H] fp32 contiguous."""
    if q.dim() != 3 or o.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("expected q, o [B, H, D] and caches [B, H, L, D]")
    B, H, L, D = (int(x) for x in k_cache.shape)
    if tuple(q.shape) != (B, H, D) or tuple(o.shape) != (B, H, D):
        raise ValueError("q and o must be [B, H, D] matching the caches")
    _same_shape(k_cache, v_cache)
    if lengths is not None:
        import torch
        if lengths.dtype != torch.int32 or tuple(lengths.shape) != (B,):
            raise ValueError("lengths must be int32 of shape [B]")
    args = []
    for t in (q.unsqueeze(2), k_cache, v_cache):
        args.extend(_sptr(t))
    args.append(_ptr(lengths))
    args.extend(_sptr(o.unsqueeze(2)))
    st = load_library().gpt_attn_decode(_dtype_code(q), B, H, L, D, *args, _ptr(lse),
                                        _ptr(workspace), _ws_bytes(workspace),
                                        _stream(q.device, stream))
    if st != 0:
        raise GptAttnError("gpt_attn_decode", st)


def attention_decode(q, k_cache, v_cache, lengths=None, stream=None, out=None, workspace=None):
    """One new query per (sequence, head) against the first lengths[b] rows
    of the caches. Allocates O (unless ``out``), LSE and the workspace;
    returns (o, lse)."""
    import torch
    B, H, L, D = (int(x) for x in k_cache.shape)
    o = torch.empty((B, H, D), dtype=q.dtype, device=q.device) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = gpt_attn_decode_workspace_bytes(_dtype_code(q), B, H, L, D)
        workspace = torch.empty(max(1, (nbytes + 3) // 4), dtype=torch.float32, device=q.device)
    gpt_attn_decode(q, k_cache, v_cache, lengths, o, lse, workspace, stream)
    return o, lse


# ---- views of the fused projection layout ---------------------------------------

def split_qkv_heads(qkv, n_head: int):
    """[B, T, 3C] projection output -> q, k, v as [B, H, T, D] views (no copy):
    the layer's single linear map produces q, k, v for every token, split
    into n_head groups of D = C / n_head."""
    if qkv.dim() != 3 or qkv.shape[2] % (3 * n_head):
        raise ValueError(f"expected [B, T, 3C] with C divisible by {n_head}")
    B, T, C3 = qkv.shape
    C = C3 // 3
    return tuple(t.view(B, T, n_head, C // n_head).transpose(1, 2)
                 for t in qkv.split(C, dim=2))


def merged_heads_view(y, n_head: int):
    """[B, T, C] buffer -> the [B, H, T, D] view that writes heads merged back."""
    if y.dim() != 3 or y.shape[2] % n_head:
        raise ValueError(f"expected [B, T, C] with C divisible by {n_head}")
    B, T, C = y.shape
    return y.view(B, T, n_head, C // n_head).transpose(1, 2)


def attention_forward(q, k, v, stream=None, keep_o_lo: bool = True, out=None, dropout=None):
    """Run the forward on [B, H, T, D] views (any layout with unit D stride).
    O goes to ``out`` (a view of that shape, e.g. merged_heads_view of a
    [B, T, C] buffer) or a new contiguous tensor; LSE (fp32) and, for bf16
    with keep_o_lo, the low part o_lo are allocated. ``dropout`` = None or
    (p, seed, offset) applies attention dropout. Returns (o, lse, o_lo)."""
    import torch
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v must share shape and dtype")
    shape = tuple(q.shape)
    o = torch.empty(shape, dtype=q.dtype, device=q.device) if out is None else out
    o_lo = (torch.empty(shape, dtype=q.dtype, device=q.device)
            if (keep_o_lo and q.dtype != torch.float32) else None)
    lse = torch.empty(shape[:-1], dtype=torch.float32, device=q.device)
    gpt_attn_fwd_strided(q, k, v, o, o_lo, lse, stream, dropout)
    return o, lse, o_lo


def attention_backward(q, k, v, o, dout, lse, o_lo=None, stream=None, workspace=None,
                       grads=None, dropout=None):
    """Run the backward on [B, H, T, D] views (any layout with unit D stride).
    dQ, dK, dV (fp32) go to ``grads`` = (dq, dk, dv) views when given (e.g.
    split_qkv_heads of an fp32 [B, T, 3C] buffer), else to new tensors; the
    workspace is allocated unless given; ``dropout`` must be the forward's.
    Returns (dq, dk, dv)."""
    import torch
    B, H, T, D = _bhtd(q)
    if grads is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        dk = torch.empty_like(dq)
        dv = torch.empty_like(dq)
    else:
        dq, dk, dv = grads
    if workspace is None:
        nbytes = gpt_attn_bwd_workspace_bytes(B, H, T, D)
        workspace = torch.empty(max(1, (nbytes + 3) // 4), dtype=torch.float32, device=q.device)
    gpt_attn_bwd_strided(q, k, v, o, o_lo, dout, lse, dq, dk, dv, workspace, stream, dropout)
    return dq, dk, dv
