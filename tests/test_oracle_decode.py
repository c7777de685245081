"""Pins for the oracle's one-query-against-a-cache function (attn_decode).

Definition (attn_oracle.c): sampling feeds the sequence back one position at
a time (generate(), page "nanoGPT: a real GPT in two 300-line files",
section 2 "How the code works"); the newest query attends to the first n
cached keys and values, n including its own position, exactly the last row
of the causal forward at T = n.

Pins: the last row of the already pinned causal forward (which is pinned to
brute force, finite differences and the library routine), the 50-digit brute
force's last row, closed forms (n = 1, n = 0), cache rows past n ignored
(NaN there changes nothing), and per-head lengths.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from tests.brute_decimal import brute_head


def _rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("n,D", [(1, 4), (2, 3), (17, 8), (64, 64), (300, 64)])
def test_equals_last_row_of_causal_forward(n, D):
    r = _rng(n + D)
    seq_q = r.standard_normal((n, D)) * 1.5
    k = r.standard_normal((n, D)) * 1.5
    v = r.standard_normal((n, D))
    o_full, lse_full = oracle.attn_fwd(seq_q, k, v)
    o, lse = oracle.attn_decode(seq_q[-1][None], k[None], v[None], [n])
    np.testing.assert_allclose(o[0], o_full[-1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], lse_full[-1], rtol=0, atol=1e-14)


@pytest.mark.parametrize("n,D", [(1, 1), (3, 2), (6, 5)])
def test_brute_force_last_row(n, D):
    r = _rng(7 * n + D)
    qs = r.standard_normal((n, D))
    k = r.standard_normal((n, D))
    v = r.standard_normal((n, D))
    ref = brute_head(qs, k, v, np.zeros((n, D)))
    o, lse = oracle.attn_decode(qs[-1][None], k[None], v[None], [n])
    np.testing.assert_allclose(o[0], ref["O"][-1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0], ref["LSE"][-1], rtol=0, atol=1e-13)


def test_closed_forms():
    r = _rng(3)
    q = r.standard_normal((2, 8))
    k = r.standard_normal((2, 5, 8))
    v = r.standard_normal((2, 5, 8))
    o, lse = oracle.attn_decode(q, k, v, [1, 0])
    assert np.array_equal(o[0], v[0, 0])                     # one key: its value
    assert math.isclose(lse[0], float(q[0] @ k[0, 0]) / math.sqrt(8), rel_tol=0, abs_tol=1e-15)
    assert not o[1].any() and lse[1] == -np.inf               # no key at all


def test_rows_past_length_are_ignored_and_lengths_per_head():
    r = _rng(11)
    B, H, L, D = 3, 2, 40, 16
    q = r.standard_normal((B, H, D))
    k = r.standard_normal((B, H, L, D))
    v = r.standard_normal((B, H, L, D))
    lengths = [40, 1, 23]
    o, lse = oracle.attn_decode(q, k, v, lengths)
    k2, v2 = k.copy(), v.copy()
    for b, n in enumerate(lengths):
        k2[b, :, n:] = np.nan
        v2[b, :, n:] = np.nan
    o2, lse2 = oracle.attn_decode(q, k2, v2, lengths)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    for b, n in enumerate(lengths):
        for h in range(H):
            ob, lb = oracle.attn_decode(q[b, h][None], k[b, h, :n][None], v[b, h, :n][None], [n])
            np.testing.assert_allclose(o[b, h], ob[0], rtol=0, atol=0)
            np.testing.assert_allclose(lse[b, h], lb[0], rtol=0, atol=0)


def test_rejects_lengths_outside_the_cache():
    z = np.zeros((1, 4))
    with pytest.raises(RuntimeError):
        oracle.attn_decode(z, np.zeros((1, 3, 4)), np.zeros((1, 3, 4)), [4])
    with pytest.raises(RuntimeError):
        oracle.attn_decode(z, np.zeros((1, 3, 4)), np.zeros((1, 3, 4)), [-1])
