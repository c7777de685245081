"""fp64 CPU oracle for causal multi-head self-attention (forward and backward).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library or its binding.
It shares no code with the GPU path. The arithmetic lives in
``attn_oracle.c`` (plain C, fp64, libm exp/log); this module only builds,
loads and marshals numpy arrays into it.

Definition followed: the slow written-out attention of nanoGPT's model.py
(page "nanoGPT: a real GPT in two 300-line files", section 2 "How the code
works": q @ k^T, times 1/sqrt(head size), future filled with -inf, softmax,
then @ v) with the causal rule of section 8 "Self-check" (a position sees
itself and earlier positions), and the analytic gradient of sum(dO * O) that
autograd forms (section 1 "Summary").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_DP = ctypes.POINTER(ctypes.c_double)


def build(verbose: bool = False) -> str:
    """Compile attn_oracle.c into liboracle.so with gcc (no fast-math, no FMA
    contraction, so every sum is evaluated exactly as written)."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c99",
           "-shared", "-fPIC", "-pthread", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    L, I = ctypes.c_long, ctypes.c_int
    lib.oracle_attn_fwd.argtypes = [L, L, L, _DP, _DP, _DP, _DP, _DP, I]
    lib.oracle_attn_fwd.restype = I
    lib.oracle_attn_bwd.argtypes = [L, L, L, _DP, _DP, _DP, _DP, _DP, _DP, _DP, I]
    lib.oracle_attn_bwd.restype = I
    lib.oracle_attn_head_intermediates.argtypes = [L, L, _DP, _DP, _DP, _DP, _DP, _DP,
                                                   _DP, _DP]
    lib.oracle_attn_head_intermediates.restype = I
    U32P = ctypes.POINTER(ctypes.c_uint32)
    U8P = ctypes.POINTER(ctypes.c_uint8)
    LP = ctypes.POINTER(ctypes.c_long)
    lib.oracle_philox4x32_10.argtypes = [U32P, U32P, U32P]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_dropout_threshold.argtypes = [ctypes.c_double]
    lib.oracle_dropout_threshold.restype = L
    lib.oracle_dropout_keep.argtypes = [L, LP, L, ctypes.c_double, ctypes.c_uint64,
                                        ctypes.c_uint32, U8P]
    lib.oracle_dropout_keep.restype = I
    lib.oracle_attn_fwd_dropout.argtypes = [L, L, L, _DP, _DP, _DP, U8P, ctypes.c_double, _DP,
                                            _DP, I]
    lib.oracle_attn_fwd_dropout.restype = I
    lib.oracle_attn_bwd_dropout.argtypes = [L, L, L, _DP, _DP, _DP, _DP, U8P, ctypes.c_double,
                                            _DP, _DP, _DP, I]
    lib.oracle_attn_bwd_dropout.restype = I
    lib.oracle_attn_decode.argtypes = [L, L, L, _DP, _DP, _DP, LP, _DP, _DP]
    lib.oracle_attn_decode.restype = I
    _lib = lib
    return lib


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: widen exactly to fp64 on the CPU
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_DP)


def _default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _heads_shape(q: np.ndarray):
    if q.ndim < 2:
        raise ValueError("expected [..., T, D]")
    T, D = q.shape[-2], q.shape[-1]
    heads = int(np.prod(q.shape[:-2])) if q.ndim > 2 else 1
    return heads, T, D


def attn_fwd(q, k, v, nthreads: int | None = None):
    """Return (O, LSE) in fp64 for inputs shaped [..., T, D]."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v shapes differ")
    heads, T, D = _heads_shape(q)
    o = np.zeros(q.shape, dtype=np.float64)
    lse = np.zeros(q.shape[:-1], dtype=np.float64)
    st = _load().oracle_attn_fwd(heads, T, D, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                 nthreads or _default_threads())
    if st != 0:
        raise RuntimeError(f"oracle_attn_fwd failed with status {st}")
    return o, lse


def attn_bwd(q, k, v, dout, nthreads: int | None = None):
    """Return (dQ, dK, dV) in fp64: the gradient of sum(dout * O)."""
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    if not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("q, k, v, dout shapes differ")
    heads, T, D = _heads_shape(q)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(q.shape, dtype=np.float64)
    dv = np.zeros(q.shape, dtype=np.float64)
    st = _load().oracle_attn_bwd(heads, T, D, _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                 _ptr(dq), _ptr(dk), _ptr(dv), nthreads or _default_threads())
    if st != 0:
        raise RuntimeError(f"oracle_attn_bwd failed with status {st}")
    return dq, dk, dv


def head_intermediates(q, k, v, dout) -> dict:
    """One head ([T, D] inputs): full T x T P, dP, dS and delta [T]."""
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    if q.ndim != 2:
        raise ValueError("expected one head [T, D]")
    T, D = q.shape
    P = np.zeros((T, T))
    dP = np.zeros((T, T))
    dS = np.zeros((T, T))
    delta = np.zeros(T)
    st = _load().oracle_attn_head_intermediates(T, D, _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                                _ptr(P), _ptr(dP), _ptr(dS), _ptr(delta))
    if st != 0:
        raise RuntimeError(f"oracle_attn_head_intermediates failed with status {st}")
    return {"P": P, "dP": dP, "dS": dS, "delta": delta}


# ---- attention dropout ------------------------------------------------------------
# Definitions in attn_oracle.c: keep mask M from Philox4x32-10 keyed by the
# seed, counter (j div 8, i, b*H + h, offset); Pd = z M P with
# z = 65536 / (65536 - thr), thr = round(p * 65536).

def philox4x32_10(counter, key) -> tuple:
    """One Philox4x32-10 block: four 32-bit outputs for a 4-word counter and a
    2-word key."""
    lib = _load()
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in counter])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    out = (ctypes.c_uint32 * 4)()
    lib.oracle_philox4x32_10(c, k, out)
    return tuple(int(x) for x in out)


def dropout_threshold(p: float) -> int:
    """thr = round(p * 65536); raises for p outside [0, 1) or thr = 65536."""
    thr = int(_load().oracle_dropout_threshold(float(p)))
    if thr < 0:
        raise ValueError(f"dropout probability {p} not in [0, 1) at 16-bit resolution")
    return thr


def dropout_scale(p: float) -> float:
    """z = 1 / (1 - thr/65536)."""
    thr = dropout_threshold(p)
    return 65536.0 / (65536.0 - thr)


def dropout_keep(heads, T: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Keep mask (uint8, 1 = kept, zero above the diagonal) of shape
    [len(heads), T, T] for the flat head indices b*H + h in ``heads``."""
    bh = np.ascontiguousarray(np.asarray(list(heads), dtype=np.int64))
    n = int(bh.size)
    keep = np.zeros((n, T, T), dtype=np.uint8)
    st = _load().oracle_dropout_keep(n, bh.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), T,
                                     float(p), int(seed) & (2**64 - 1),
                                     int(offset) & 0xFFFFFFFF,
                                     keep.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    if st != 0:
        raise RuntimeError(f"oracle_dropout_keep failed with status {st}")
    return keep


def _keep_arg(keep, heads: int, T: int) -> np.ndarray:
    keep = np.ascontiguousarray(np.asarray(keep, dtype=np.uint8))
    if keep.size != heads * T * T:
        raise ValueError(f"keep mask must hold {heads} x {T} x {T} entries")
    return keep


def attn_fwd_dropout(q, k, v, keep, z: float, nthreads: int | None = None):
    """(O, LSE) in fp64 with attention dropout given by the explicit keep mask
    [heads, T, T] and survivor scale z."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v shapes differ")
    heads, T, D = _heads_shape(q)
    keep = _keep_arg(keep, heads, T)
    o = np.zeros(q.shape, dtype=np.float64)
    lse = np.zeros(q.shape[:-1], dtype=np.float64)
    st = _load().oracle_attn_fwd_dropout(
        heads, T, D, _ptr(q), _ptr(k), _ptr(v),
        keep.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), float(z), _ptr(o), _ptr(lse),
        nthreads or _default_threads())
    if st != 0:
        raise RuntimeError(f"oracle_attn_fwd_dropout failed with status {st}")
    return o, lse


def attn_bwd_dropout(q, k, v, dout, keep, z: float, nthreads: int | None = None):
    """(dQ, dK, dV) in fp64: the gradient of sum(dout * O) for attn_fwd_dropout."""
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    if not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("q, k, v, dout shapes differ")
    heads, T, D = _heads_shape(q)
    keep = _keep_arg(keep, heads, T)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(q.shape, dtype=np.float64)
    dv = np.zeros(q.shape, dtype=np.float64)
    st = _load().oracle_attn_bwd_dropout(
        heads, T, D, _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
        keep.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), float(z), _ptr(dq), _ptr(dk),
        _ptr(dv), nthreads or _default_threads())
    if st != 0:
        raise RuntimeError(f"oracle_attn_bwd_dropout failed with status {st}")
    return dq, dk, dv


# ---- one query against a key/value cache --------------------------------------------

def attn_decode(q, k, v, lengths):
    """(O [..., D], LSE [...]) in fp64 for queries q [..., D] against caches
    k, v [..., L, D] of which the first lengths[...] rows are used (lengths
    broadcast over the leading dimensions of q, e.g. [B] for q [B, H, D])."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if k.shape != v.shape or k.shape[:-2] != q.shape[:-1] or k.shape[-1] != q.shape[-1]:
        raise ValueError("expected q [..., D] and k, v [..., L, D]")
    lead = q.shape[:-1]
    L, D = k.shape[-2], k.shape[-1]
    heads = int(np.prod(lead)) if lead else 1
    lens = np.asarray(lengths, dtype=np.int64)
    while lens.ndim < len(lead):
        lens = lens[..., None]
    lens = np.ascontiguousarray(np.broadcast_to(lens, lead).reshape(-1))
    o = np.zeros(q.shape, dtype=np.float64)
    lse = np.zeros(lead, dtype=np.float64)
    st = _load().oracle_attn_decode(heads, L, D, _ptr(q), _ptr(k), _ptr(v),
                                    lens.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                                    _ptr(o), _ptr(lse))
    if st != 0:
        raise RuntimeError(f"oracle_attn_decode failed with status {st}")
    return o, lse
