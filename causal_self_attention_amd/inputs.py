"""Seeded synthetic inputs for causal self-attention: Q, K, V and the upstream
gradient dO, all laid out [B, H, T, D] and contiguous.

This module holds none of the attention arithmetic. It only draws standard
normal samples in a fixed order, optionally multiplies Q and K by a constant
(to sharpen the softmax) and rounds to the working dtype. Both the fp64 oracle
and the GPU path consume exactly these tensors.

Recipe (one ``torch.Generator('cpu')`` per call, seeded with ``seed``):
  1. draw Q, K, V, dO in that order with ``torch.randn(B, H, T, D, float32)``;
  2. multiply Q and K by ``qk_scale`` in fp32;
  3. cast to the working dtype (bf16 uses round-to-nearest-even).

The shapes are the attention layers of the models the nanoGPT pages train:
the "baby GPT" Shakespeare-char model (6 heads of 64 channels, block size
256), the smaller Shakespeare-char run on a laptop (4 heads of 32 channels,
block size 64, batch 12) and GPT-2 124M / 350M / 774M / 1558M (12 / 16 / 20 /
25 heads of 64, block size 1024). The pages give no activation statistics, so i.i.d. N(0, 1) draws stand
in for real activations.

Decode inputs (one new query per sequence against a key/value cache, as
sampling with generate() does one position at a time): q [B, H, D] and
caches k, v [B, H, L, D] drawn in that order with ``torch.randn`` in fp32,
then cast; with ``ragged`` the per-sequence lengths [B] are drawn uniformly
from 1 .. L with ``torch.randint`` from the same generator afterwards,
otherwise every length is L.
"""
from __future__ import annotations

import dataclasses

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "workload_inputs", "torch_dtype",
           "DecodeWorkload", "DECODE_WORKLOADS", "make_decode_inputs", "decode_inputs"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-layer shape with its input dtype and Q/K draw scale."""

    name: str
    dtype: str  # "f32", "bf16" or "f16"
    B: int
    H: int
    T: int
    D: int
    qk_scale: float = 1.0


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in (
        # Shakespeare-char "baby GPT" layer in fp32, batch 1.
        Workload("shakespeare_char_f32_b1_h6_t256", "f32", 1, 6, 256, 64),
        # Same layer at the training batch of 64, bf16 in / fp32 accumulate.
        Workload("shakespeare_char_bf16_b64_h6_t256", "bf16", 64, 6, 256, 64),
        # GPT-2 124M attention layer.
        Workload("gpt2_124m_bf16_b12_h12_t1024", "bf16", 12, 12, 1024, 64),
        # GPT-2 350M attention layer (16 heads of 64, block 1024) at the same
        # batch of 12 sequences.
        Workload("gpt2_350m_bf16_b12_h16_t1024", "bf16", 12, 16, 1024, 64),
        # GPT-2 774M attention layer with Q, K drawn at std 2 (sharper softmax).
        Workload("gpt2_774m_sharp_bf16_b8_h20_t1024", "bf16", 8, 20, 1024, 64, 2.0),
        # GPT-2 1558M attention layer, and the same heads at twice the context.
        Workload("gpt2_1558m_bf16_b4_h25_t1024", "bf16", 4, 25, 1024, 64),
        Workload("gpt2_1558m_long_bf16_b2_h25_t2048", "bf16", 2, 25, 2048, 64),
        # GPT-2 124M layer under fp16 mixed precision.
        Workload("gpt2_124m_f16_b12_h12_t1024", "f16", 12, 12, 1024, 64),
        # The laptop Shakespeare-char run: batch 12, 4 heads of 32 channels,
        # block 64 (head size 128 / 4), in fp32 and bf16.
        Workload("shakespeare_char_small_f32_b12_h4_t64_d32", "f32", 12, 4, 64, 32),
        Workload("shakespeare_char_small_bf16_b12_h4_t64_d32", "bf16", 12, 4, 64, 32),
        # Head size 128 (not a model of the pages; the head size of larger
        # models): the GPT-2 774M layer's width, 1280 channels, as 10 heads of
        # 128 instead of 20 of 64.
        Workload("gpt2_774m_d128_bf16_b8_h10_t1024", "bf16", 8, 10, 1024, 128),
    )
}


def torch_dtype(dtype: str) -> torch.dtype:
    if dtype == "f32":
        return torch.float32
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f16":
        return torch.float16
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(B: int, H: int, T: int, D: int, dtype: str = "bf16", seed: int = 0,
                qk_scale: float = 1.0) -> dict[str, torch.Tensor]:
    """Return CPU tensors ``q, k, v, do`` of shape [B, H, T, D] in ``dtype``."""
    gen = torch.Generator("cpu").manual_seed(seed)
    shape = (B, H, T, D)
    q = torch.randn(shape, dtype=torch.float32, generator=gen)
    k = torch.randn(shape, dtype=torch.float32, generator=gen)
    v = torch.randn(shape, dtype=torch.float32, generator=gen)
    do = torch.randn(shape, dtype=torch.float32, generator=gen)
    if qk_scale != 1.0:
        q = q * qk_scale
        k = k * qk_scale
    td = torch_dtype(dtype)
    return {"q": q.to(td).contiguous(), "k": k.to(td).contiguous(),
            "v": v.to(td).contiguous(), "do": do.to(td).contiguous()}


def workload_inputs(w: Workload, seed: int = 0) -> dict[str, torch.Tensor]:
    return make_inputs(w.B, w.H, w.T, w.D, w.dtype, seed, w.qk_scale)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode step of an attention layer: B sequences, cache length L."""

    name: str
    dtype: str
    B: int
    H: int
    L: int
    D: int
    ragged: bool = False


DECODE_WORKLOADS: dict[str, DecodeWorkload] = {
    w.name: w
    for w in (
        # GPT-2 124M layer sampling 64 sequences at a full 1024-token context.
        DecodeWorkload("gpt2_124m_decode_bf16_b64_h12_l1024", "bf16", 64, 12, 1024, 64),
        # The same with every sequence at its own length in 1 .. 1024.
        DecodeWorkload("gpt2_124m_decode_ragged_bf16_b64_h12_l1024", "bf16", 64, 12, 1024, 64,
                       True),
        # Shakespeare-char layer sampling one sequence (block size 256), fp32.
        DecodeWorkload("shakespeare_char_decode_f32_b1_h6_l256", "f32", 1, 6, 256, 64),
    )
}


def make_decode_inputs(B: int, H: int, L: int, D: int, dtype: str = "bf16", seed: int = 0,
                       ragged: bool = False) -> dict[str, torch.Tensor]:
    """CPU tensors q [B, H, D], k, v [B, H, L, D] in ``dtype`` and lengths
    [B] (int32)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, H, D), dtype=torch.float32, generator=gen)
    k = torch.randn((B, H, L, D), dtype=torch.float32, generator=gen)
    v = torch.randn((B, H, L, D), dtype=torch.float32, generator=gen)
    if ragged and L > 0:
        lengths = torch.randint(1, L + 1, (B,), generator=gen, dtype=torch.int64)
    else:
        lengths = torch.full((B,), L, dtype=torch.int64)
    td = torch_dtype(dtype)
    return {"q": q.to(td).contiguous(), "k": k.to(td).contiguous(),
            "v": v.to(td).contiguous(), "lengths": lengths.to(torch.int32)}


def decode_inputs(w: DecodeWorkload, seed: int = 0) -> dict[str, torch.Tensor]:
    return make_decode_inputs(w.B, w.H, w.L, w.D, w.dtype, seed, w.ragged)
