"""Pins for the fp64 oracle, each independent of the oracle's own code.

Definition pinned: causal softmax attention as nanoGPT's slow written-out
path computes it (page "nanoGPT: a real GPT in two 300-line files", section 2
"How the code works"; causality per section 8 "Self-check") and its analytic
gradient (section 1 "Summary": autograd supplies it).

Pins: hand-derived closed-form fixtures (tests/golden), 50-digit brute force
with the explicit softmax Jacobian, central finite differences, the library
routine the pages name (scaled_dot_product_attention, is_causal=True) in fp64
with autograd, special cases with closed forms (row 0, T = 1, all keys equal,
Q = 0), the zero row sums of dS, the column sums of dK and dV, and
equivariances (value shift, key shift, head slicing).
"""
from __future__ import annotations

import ast
import json
import math
import os
import operator

import numpy as np
import pytest
import torch

import oracle
from tests.brute_decimal import brute_head

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_examples.json")


def rng_inputs(B, H, T, D, seed, scale=1.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, D)) * scale
    k = r.standard_normal((B, H, T, D)) * scale
    v = r.standard_normal((B, H, T, D))
    do = r.standard_normal((B, H, T, D))
    return q, k, v, do


# ---- closed-form fixtures ---------------------------------------------------

_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv, ast.USub: operator.neg}


def _eval_expr(text: str) -> float:
    """Evaluate a fixture expression: numbers, + - * /, unary minus, ln(n)."""
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.BinOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](ev(node.left), ev(node.right))
        if isinstance(node, ast.UnaryOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](ev(node.operand))
        if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name)
                and node.func.id == "ln" and len(node.args) == 1):
            return math.log(ev(node.args[0]))
        raise ValueError(f"unsupported fixture expression: {text!r}")
    return ev(ast.parse(text, mode="eval"))


def _arr(rows):
    if isinstance(rows[0], list):
        return np.array([[_eval_expr(x) for x in r] for r in rows])
    return np.array([_eval_expr(x) for x in rows])


def _golden_examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _golden_examples(), ids=lambda e: e["name"])
def test_closed_form_fixture(ex):
    T, D = ex["T"], ex["D"]
    assert abs(1.0 / math.sqrt(D) - _eval_expr(ex["scale"])) == 0.0
    q, k, v, do = (_arr(ex[n]) for n in ("q", "k", "v", "do"))
    assert q.shape == (T, D)
    o, lse = oracle.attn_fwd(q, k, v)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do)
    np.testing.assert_allclose(o, _arr(ex["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, _arr(ex["lse"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dq, _arr(ex["dq"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk, _arr(ex["dk"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv, _arr(ex["dv"]), rtol=0, atol=1e-14)


# ---- brute force --------------------------------------------------------------

BRUTE_SHAPES = [(1, 1, 1, 1), (1, 1, 2, 1), (2, 1, 3, 2), (1, 2, 5, 3), (1, 1, 9, 12),
                (1, 1, 4, 64), (2, 2, 7, 3), (1, 1, 8, 2)]


@pytest.mark.parametrize("shape", BRUTE_SHAPES, ids=str)
def test_brute_force_decimal(shape):
    B, H, T, D = shape
    q, k, v, do = rng_inputs(B, H, T, D, seed=sum(shape), scale=1.5)
    o, lse = oracle.attn_fwd(q, k, v)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do)
    for b in range(B):
        for h in range(H):
            ref = brute_head(q[b, h], k[b, h], v[b, h], do[b, h])
            np.testing.assert_allclose(o[b, h], ref["O"], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], ref["LSE"], rtol=0, atol=1e-12)
            np.testing.assert_allclose(dq[b, h], ref["dQ"], rtol=0, atol=1e-12)
            np.testing.assert_allclose(dk[b, h], ref["dK"], rtol=0, atol=1e-12)
            np.testing.assert_allclose(dv[b, h], ref["dV"], rtol=0, atol=1e-12)
            P = oracle.head_intermediates(q[b, h], k[b, h], v[b, h], do[b, h])["P"]
            np.testing.assert_allclose(P, ref["P"], rtol=0, atol=1e-13)


# ---- finite differences -----------------------------------------------------

@pytest.mark.parametrize("shape", [(1, 1, 5, 3), (1, 2, 6, 4), (1, 1, 9, 8)], ids=str)
def test_central_finite_differences(shape):
    """Gradient of L = sum(dO * O) by central differences, h = 1e-5; per
    tensor, max |fd - an| / max |an| <= 1e-6."""
    B, H, T, D = shape
    q, k, v, do = rng_inputs(B, H, T, D, seed=7 + T)
    an = dict(zip("qkv", oracle.attn_bwd(q, k, v, do)))
    h = 1e-5
    base = {"q": q, "k": k, "v": v}
    for name in "qkv":
        x = base[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = {n: a.copy() for n, a in base.items()}
            args[name][idx] += h
            lp = np.sum(do * oracle.attn_fwd(args["q"], args["k"], args["v"])[0])
            args[name][idx] -= 2 * h
            lm = np.sum(do * oracle.attn_fwd(args["q"], args["k"], args["v"])[0])
            fd[idx] = (lp - lm) / (2 * h)
        rel = np.max(np.abs(fd - an[name])) / np.max(np.abs(an[name]))
        assert rel <= 1e-6, (name, rel)


# ---- the library routine the pages name -------------------------------------

@pytest.mark.parametrize("shape", [(2, 3, 37, 16), (1, 2, 128, 64), (1, 1, 1, 64)], ids=str)
def test_matches_torch_sdpa_fp64(shape):
    """scaled_dot_product_attention(q, k, v, is_causal=True), the call nanoGPT
    makes, evaluated in fp64 on the CPU with autograd."""
    B, H, T, D = shape
    q, k, v, do = rng_inputs(B, H, T, D, seed=3, scale=2.0)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=None,
                                                           dropout_p=0.0, is_causal=True)
    out.backward(torch.tensor(do))
    o, _ = oracle.attn_fwd(q, k, v)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do)
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


# ---- closed forms -------------------------------------------------------------

def test_row_zero_exact():
    q, k, v, do = rng_inputs(2, 3, 17, 64, seed=11)
    o, lse = oracle.attn_fwd(q, k, v)
    dq, _, _ = oracle.attn_bwd(q, k, v, do)
    assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :])
    s00 = np.einsum("bhd,bhd->bh", q[:, :, 0, :], k[:, :, 0, :]) / 8.0
    np.testing.assert_allclose(lse[:, :, 0], s00, rtol=1e-14, atol=1e-14)
    assert np.all(dq[:, :, 0, :] == 0.0)


def test_single_position():
    q, k, v, do = rng_inputs(3, 2, 1, 64, seed=5)
    o, lse = oracle.attn_fwd(q, k, v)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do)
    assert np.array_equal(o, v)
    assert np.array_equal(dv, do)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    np.testing.assert_allclose(lse[..., 0], np.sum(q[..., 0, :] * k[..., 0, :], -1) / 8.0,
                               rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("zero_q", [False, True])
def test_uniform_attention(zero_q):
    """All keys equal (or Q = 0): P_ij = 1/(i+1), so O_t = mean(V_0..V_t),
    LSE_t = S_t0 + ln(t+1) and dV_j = sum_{i>=j} dO_i/(i+1). Equal keys give
    dQ = 0 (each row of dS sums to zero); Q = 0 gives dK = 0."""
    B, H, T, D = 1, 2, 23, 16
    q, k, v, do = rng_inputs(B, H, T, D, seed=9)
    if zero_q:
        q[:] = 0.0
    else:
        k[:] = k[:, :, :1, :]
    o, lse = oracle.attn_fwd(q, k, v)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do)
    counts = np.arange(1, T + 1)[:, None]
    mean_v = np.cumsum(v, axis=2) / counts
    np.testing.assert_allclose(o, mean_v, rtol=0, atol=1e-13)
    s_t0 = np.sum(q * k[:, :, :1, :], -1) / math.sqrt(D)
    np.testing.assert_allclose(lse, s_t0 + np.log(np.arange(1, T + 1)), rtol=0, atol=1e-13)
    w = do / counts  # dO_i / (i+1)
    dv_ref = np.flip(np.cumsum(np.flip(w, axis=2), axis=2), axis=2)
    np.testing.assert_allclose(dv, dv_ref, rtol=0, atol=1e-13)
    if zero_q:
        np.testing.assert_allclose(dk, 0.0, rtol=0, atol=1e-13)
    else:
        np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-13)


def test_probability_rows_and_zero_score_gradient_rows():
    q, k, v, do = rng_inputs(1, 1, 31, 8, seed=13, scale=2.0)
    r = oracle.head_intermediates(q[0, 0], k[0, 0], v[0, 0], do[0, 0])
    P, dP, dS = r["P"], r["dP"], r["dS"]
    assert np.all(np.triu(P, 1) == 0.0) and np.all(P >= 0.0)
    np.testing.assert_allclose(P.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.abs(dS.sum(1)) <= 1e-12 * np.max(np.abs(dP)))
    assert np.all(np.triu(dS, 1) == 0.0)


def test_column_sums():
    """Per head: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i."""
    q, k, v, do = rng_inputs(2, 2, 40, 12, seed=17, scale=1.5)
    _, dk, dv = oracle.attn_bwd(q, k, v, do)
    np.testing.assert_allclose(dk.sum(2), 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(2), do.sum(2), rtol=0, atol=1e-12)


# ---- equivariances -------------------------------------------------------------

def test_value_affine_equivariance():
    q, k, v, _ = rng_inputs(1, 2, 19, 8, seed=21)
    alpha, beta = -1.75, np.linspace(-2, 3, 8)
    o1, l1 = oracle.attn_fwd(q, k, v)
    o2, l2 = oracle.attn_fwd(q, k, alpha * v + beta)
    np.testing.assert_allclose(o2, alpha * o1 + beta, rtol=0, atol=1e-13)
    assert np.array_equal(l1, l2)


def test_key_shift():
    """K -> K + 1 c^T shifts every score in row i by s Q_i . c: O is unchanged
    and LSE_i moves by s Q_i . c."""
    q, k, v, _ = rng_inputs(1, 2, 19, 8, seed=23)
    c = np.linspace(1.0, -0.5, 8)
    o1, l1 = oracle.attn_fwd(q, k, v)
    o2, l2 = oracle.attn_fwd(q, k + c, v)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + (q @ c) / math.sqrt(8), rtol=0, atol=1e-13)


def test_head_slicing_and_thread_count():
    q, k, v, do = rng_inputs(3, 4, 21, 16, seed=29)
    o, lse = oracle.attn_fwd(q, k, v, nthreads=5)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, nthreads=3)
    o1, lse1 = oracle.attn_fwd(q, k, v, nthreads=1)
    assert np.array_equal(o, o1) and np.array_equal(lse, lse1)
    b, h = 2, 1
    os_, ls_ = oracle.attn_fwd(q[b, h], k[b, h], v[b, h])
    g = oracle.attn_bwd(q[b, h], k[b, h], v[b, h], do[b, h], nthreads=1)
    assert np.array_equal(os_, o[b, h]) and np.array_equal(ls_, lse[b, h])
    for a, full in zip(g, (dq, dk, dv)):
        assert np.array_equal(a, full[b, h])


def test_causality_future_inputs_do_not_leak():
    """Changing K, V at positions > t leaves O and LSE of rows <= t unchanged."""
    q, k, v, _ = rng_inputs(1, 1, 16, 8, seed=31)
    o1, l1 = oracle.attn_fwd(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[..., 9:, :] += 5.0
    v2[..., 9:, :] -= 3.0
    o2, l2 = oracle.attn_fwd(q, k2, v2)
    assert np.array_equal(o1[..., :9, :], o2[..., :9, :])
    assert np.array_equal(l1[..., :9], l2[..., :9])
    assert not np.allclose(o1[..., 9:, :], o2[..., 9:, :])


def test_empty_inputs():
    z = np.zeros((2, 3, 0, 64))
    o, lse = oracle.attn_fwd(z, z, z)
    assert o.shape == z.shape and lse.shape == (2, 3, 0)
    g = oracle.attn_bwd(z, z, z, z)
    assert all(a.shape == z.shape for a in g)
