"""Pins for the oracle's attention dropout, each independent of its code.

Definition pinned (attn_oracle.c): nanoGPT hands its dropout rate to the
fused attention call in training (page "nanoGPT: a real GPT in two 300-line
files", section 2 "How the code works"): weights are zeroed with probability
p after the softmax and the survivors scaled so the expectation is unchanged.
The keep mask comes from Philox4x32-10 (Salmon et al., SC'11) keyed by the
seed, with counter (j div 8, i, b*H + h, offset) and the 16-bit field of key
j in the block's output.

Pins:
  * the generator against rocRAND's Philox4x32-10 engine (a library routine,
    compiled on the host from the ROCm headers), for every counter and key
    word, and the whole mask mapping recomputed from rocRAND's outputs;
  * the threshold rule at hand-computed values and at its boundary;
  * mask statistics (drop rate, no correlation between neighbours, distinct
    streams per head / offset / seed);
  * attention with a mask against the 50-digit brute force (explicit chain
    rule through the full dropped matrix), central finite differences, p = 0
    against the plain oracle, closed forms (everything dropped, only the
    diagonal kept), and the Monte Carlo expectation over masks.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from tests.brute_decimal import brute_head

HERE = os.path.dirname(os.path.abspath(__file__))
REF_SRC = os.path.join(HERE, "rocrand_philox_ref.cpp")
MASK64 = 2**64 - 1


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def build_rocrand_ref(out_dir):
    """Compile the rocRAND reference program into out_dir; return a callable
    list of (seed, subsequence, offset) -> list of 4-word blocks, or None when
    hipcc or the rocRAND headers are missing."""
    hipcc = _hipcc()
    if hipcc is None or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        return None
    exe = os.path.join(str(out_dir), "philox_ref")
    subprocess.run([hipcc, "-O1", REF_SRC, "-o", exe], check=True, capture_output=True)

    def run(reqs):
        text = "".join(f"{s} {u} {o}\n" for s, u, o in reqs)
        out = subprocess.run([exe], input=text, capture_output=True, text=True,
                             check=True).stdout.split("\n")
        return [tuple(int(w, 16) for w in line.split()) for line in out if line.strip()]
    return run


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    run = build_rocrand_ref(tmp_path_factory.mktemp("rocrand"))
    if run is None:
        pytest.skip("hipcc / rocRAND headers not available: generator pin not run")
    return run


def _words(x):
    return x & 0xFFFFFFFF, (x >> 32) & 0xFFFFFFFF


def test_philox_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(2024)
    reqs, ours = [], []
    for n in range(200):
        seed = int(rng.integers(0, 2**63)) * 2 + int(n & 1)
        sub = int(rng.integers(0, 2**63))
        blk = int(rng.integers(0, 2**30))
        if n < 4:  # all-zero and all-ones corners of each word group
            seed, sub, blk = [(0, 0, 0), (MASK64, 0, 0), (0, MASK64, 0), (0, 0, 2**30 - 1)][n]
        reqs.append((seed, sub, 4 * blk))
        ctr = (*_words(blk), *_words(sub))
        ours.append(oracle.philox4x32_10(ctr, _words(seed)))
    assert rocrand_ref(reqs) == ours


def test_keep_mask_recomputed_from_rocrand(rocrand_ref):
    """The whole mapping (counter layout, word and 16-bit field selection,
    threshold compare) rebuilt from rocRAND's blocks on sampled entries."""
    T, p, seed, offset = 77, 0.3, 0xDEADBEEF12345, 9
    heads = [0, 3, 1234567]
    keep = oracle.dropout_keep(heads, T, p, seed, offset)
    thr = oracle.dropout_threshold(p)
    rng = np.random.default_rng(5)
    picks = []
    for hi, bh in enumerate(heads):
        for _ in range(150):
            i = int(rng.integers(0, T))
            j = int(rng.integers(0, i + 1))
            picks.append((hi, bh, i, j))
    reqs = [(seed, bh | (offset << 32), 4 * ((j // 8) | (i << 32))) for _, bh, i, j in picks]
    blocks = rocrand_ref(reqs)
    for (hi, bh, i, j), blk in zip(picks, blocks):
        u = (blk[(j % 8) // 2] >> (16 * (j % 2))) & 0xFFFF
        assert keep[hi, i, j] == (1 if u >= thr else 0), (bh, i, j, u, thr)
    # Above the diagonal nothing is kept.
    assert not np.triu(keep[0], 1).any()


def test_threshold_compare_boundary(rocrand_ref):
    """u == thr is kept, u == thr - 1 dropped: choose p from a known u."""
    seed, offset, bh, i, j = 77, 3, 2, 40, 21
    blk = rocrand_ref([(seed, bh | (offset << 32), 4 * ((j // 8) | (i << 32)))])[0]
    u = (blk[(j % 8) // 2] >> (16 * (j % 2))) & 0xFFFF
    assert 0 < u < 65535
    keep_at = oracle.dropout_keep([bh], i + 1, u / 65536.0, seed, offset)
    keep_above = oracle.dropout_keep([bh], i + 1, (u + 1) / 65536.0, seed, offset)
    assert keep_at[0, i, j] == 1 and keep_above[0, i, j] == 0


def test_threshold_values():
    # thr = round(p * 65536), computed by hand.
    assert oracle.dropout_threshold(0.0) == 0
    assert oracle.dropout_threshold(0.2) == 13107      # 13107.2
    assert oracle.dropout_threshold(0.3) == 19661      # 19660.8
    assert oracle.dropout_threshold(0.5) == 32768
    assert oracle.dropout_threshold(0.1) == 6554       # 6553.6
    assert oracle.dropout_threshold(0.99999) == 65535  # 65535.34
    for bad in (-0.1, 1.0, 0.999995, float("nan"), 2.0):
        with pytest.raises(ValueError):
            oracle.dropout_threshold(bad)
    assert oracle.dropout_scale(0.5) == 2.0
    assert oracle.dropout_scale(0.0) == 1.0


def test_mask_statistics():
    T = 400
    tri = np.tril(np.ones((T, T), dtype=bool))
    for p in (0.1, 0.2, 0.5):
        keep = oracle.dropout_keep(range(4), T, p, seed=123, offset=0)
        n = int(tri.sum()) * 4
        drop = 1.0 - keep[:, tri].mean()
        pe = oracle.dropout_threshold(p) / 65536.0
        assert abs(drop - pe) <= 5 * np.sqrt(pe * (1 - pe) / n), (p, drop)
        # Neighbouring keys and neighbouring queries are uncorrelated.
        a = keep[:, 1:, :-1][:, tri[1:, :-1]].astype(float)
        b = keep[:, 1:, 1:][:, tri[1:, :-1]].astype(float)
        c = keep[:, :-1, :-1][:, tri[1:, :-1]].astype(float)
        for x, y in ((a, b), (a, c)):
            r = np.corrcoef(x.ravel(), y.ravel())[0, 1]
            assert abs(r) < 5 / np.sqrt(x.size), r
    base = oracle.dropout_keep([0, 1], 64, 0.5, seed=1, offset=0)
    assert not np.array_equal(base[0], base[1])                       # heads differ
    assert not np.array_equal(base, oracle.dropout_keep([0, 1], 64, 0.5, 1, 1))  # offsets
    assert not np.array_equal(base, oracle.dropout_keep([0, 1], 64, 0.5, 2, 0))  # seeds
    assert np.array_equal(base, oracle.dropout_keep([0, 1], 64, 0.5, 1, 0))      # repeatable
    # A head's mask does not depend on which other heads are requested.
    assert np.array_equal(base[1], oracle.dropout_keep([1], 64, 0.5, 1, 0)[0])
    # p = 0 keeps every visible entry.
    k0 = oracle.dropout_keep([0], 50, 0.0, 9, 9)[0]
    assert np.array_equal(k0, np.tril(np.ones((50, 50), dtype=np.uint8)))


def _inputs(B, H, T, D, seed, scale=1.5):
    r = np.random.default_rng(seed)
    return tuple(r.standard_normal((B, H, T, D)) * (scale if n < 2 else 1.0) for n in range(4))


def _random_keep(heads, T, rate, seed):
    r = np.random.default_rng(seed)
    m = (r.random((heads, T, T)) >= rate).astype(np.uint8)
    return m * np.tril(np.ones((T, T), dtype=np.uint8))


@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (1, 1, 3, 2), (1, 2, 5, 3), (1, 1, 8, 4)],
                         ids=str)
def test_brute_force_decimal_with_mask(shape):
    B, H, T, D = shape
    q, k, v, do = _inputs(B, H, T, D, seed=sum(shape) + 100)
    keep = _random_keep(B * H, T, 0.4, seed=T)
    z = 1.0 / 0.6
    o, lse = oracle.attn_fwd_dropout(q, k, v, keep, z)
    dq, dk, dv = oracle.attn_bwd_dropout(q, k, v, do, keep, z)
    for h in range(B * H):
        b, hh = divmod(h, H)
        ref = brute_head(q[b, hh], k[b, hh], v[b, hh], do[b, hh], keep=keep[h], z=z)
        np.testing.assert_allclose(o[b, hh], ref["O"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b, hh], ref["LSE"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dq[b, hh], ref["dQ"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk[b, hh], ref["dK"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv[b, hh], ref["dV"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", [(1, 1, 6, 3), (1, 2, 7, 4)], ids=str)
def test_finite_differences_with_mask(shape):
    B, H, T, D = shape
    q, k, v, do = _inputs(B, H, T, D, seed=31 + T, scale=1.0)
    keep = _random_keep(B * H, T, 0.3, seed=4)
    z = 1.0 / 0.7
    an = dict(zip("qkv", oracle.attn_bwd_dropout(q, k, v, do, keep, z)))
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
            lp = np.sum(do * oracle.attn_fwd_dropout(args["q"], args["k"], args["v"], keep, z)[0])
            args[name][idx] -= 2 * h
            lm = np.sum(do * oracle.attn_fwd_dropout(args["q"], args["k"], args["v"], keep, z)[0])
            fd[idx] = (lp - lm) / (2 * h)
        rel = np.max(np.abs(fd - an[name])) / np.max(np.abs(an[name]))
        assert rel <= 1e-6, (name, rel)


def test_keep_all_equals_plain_oracle():
    q, k, v, do = _inputs(2, 2, 33, 16, seed=8)
    keep = oracle.dropout_keep(range(4), 33, 0.0, seed=5, offset=0)
    o, lse = oracle.attn_fwd_dropout(q, k, v, keep, 1.0)
    o0, lse0 = oracle.attn_fwd(q, k, v)
    assert np.array_equal(o, o0) and np.array_equal(lse, lse0)
    g = oracle.attn_bwd_dropout(q, k, v, do, keep, 1.0)
    g0 = oracle.attn_bwd(q, k, v, do)
    for a, b in zip(g, g0):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_closed_forms_all_dropped_and_diagonal_only():
    T, D = 9, 5
    q, k, v, do = _inputs(1, 1, T, D, seed=12)
    none = np.zeros((1, T, T), dtype=np.uint8)
    o, lse = oracle.attn_fwd_dropout(q, k, v, none, 1.25)
    assert not o.any()
    np.testing.assert_allclose(lse, oracle.attn_fwd(q, k, v)[1], rtol=0, atol=0)
    for g in oracle.attn_bwd_dropout(q, k, v, do, none, 1.25):
        assert not g.any()
    # Only the diagonal kept: O_i = z P_ii V_i with P_ii = exp(S_ii - LSE_i).
    diag = np.eye(T, dtype=np.uint8)[None]
    z = 1.25
    o, lse = oracle.attn_fwd_dropout(q, k, v, diag, z)
    S = np.einsum("td,td->t", q[0, 0], k[0, 0]) / np.sqrt(D)
    pii = np.exp(S - lse[0, 0])
    np.testing.assert_allclose(o[0, 0], z * pii[:, None] * v[0, 0], rtol=0, atol=1e-14)
    _, _, dv = oracle.attn_bwd_dropout(q, k, v, do, diag, z)
    np.testing.assert_allclose(dv[0, 0], z * pii[:, None] * do[0, 0], rtol=0, atol=1e-14)


def test_expectation_over_masks():
    """Averaged over many offsets, the dropped output approaches the plain one
    (E[z M] = 1); the error shrinks like 1/sqrt(samples)."""
    T, D, n = 6, 3, 3000
    q, k, v, _ = _inputs(1, 1, T, D, seed=21)
    p = 0.5
    z = oracle.dropout_scale(p)
    acc = np.zeros((T, D))
    sq = np.zeros((T, D))
    for off in range(n):
        keep = oracle.dropout_keep([0], T, p, seed=77, offset=off)
        o = oracle.attn_fwd_dropout(q, k, v, keep, z)[0][0, 0]
        acc += o
        sq += o * o
    mean = acc / n
    sd = np.sqrt(np.maximum(sq / n - mean**2, 1e-30) / n)
    o0 = oracle.attn_fwd(q, k, v)[0][0, 0]
    assert np.all(np.abs(mean - o0) <= 5 * sd + 1e-12), np.max(np.abs(mean - o0) / (sd + 1e-30))
