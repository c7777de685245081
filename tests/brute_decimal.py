"""Brute-force causal attention in 50-digit decimal arithmetic: an independent
pin for the fp64 oracle on tiny inputs.

It differs from the oracle on purpose wherever a plausible mistake could hide:
  * the full T x T score matrix is materialized, future entries set to zero
    weight (the -infinity of the causal fill, page "nanoGPT: a real GPT in two
    300-line files", section 2 "How the code works", and section 8
    "Self-check");
  * the softmax is exp(S) / sum exp(S) with no max subtraction;
  * the score gradient goes through the explicit softmax Jacobian
    J = diag(P_i) - P_i P_i^T applied to dP_i, not through
    delta = rowsum(dO * O);
  * all arithmetic is Python ``decimal`` at 50 significant digits, seeded
    with the exact binary values of the fp64 inputs.

With a keep mask M and survivor scale z (attention dropout: the weights are
zeroed where M is 0 and scaled by z elsewhere, after the softmax; same page,
section 2), the dropped matrix Pd = z M P is formed in full and the chain
rule runs through it: dPd = dO V^T, dP = z M dPd, then the Jacobian.
"""
from __future__ import annotations

from decimal import Decimal, localcontext


def _dec(rows):
    return [[Decimal(float(x)) for x in r] for r in rows]


def brute_head(q, k, v, do, prec: int = 50, keep=None, z=1.0):
    """One head ([T][D] nested sequences). Returns a dict of float lists:
    O [T][D], LSE [T], dQ, dK, dV [T][D], P [T][T]. ``keep`` ([T][T] of 0/1)
    and ``z`` apply attention dropout."""
    with localcontext() as ctx:
        ctx.prec = prec
        Q, K, V, dO = _dec(q), _dec(k), _dec(v), _dec(do)
        T, D = len(Q), len(Q[0])
        s = Decimal(1) / Decimal(D).sqrt()
        zero = Decimal(0)
        # Full score matrix, every (i, j) including the future.
        S = [[s * sum((Q[i][d] * K[j][d] for d in range(D)), zero) for j in range(T)]
             for i in range(T)]
        # Causal weights: exp of visible scores, exactly zero for j > i.
        E = [[S[i][j].exp() if j <= i else zero for j in range(T)] for i in range(T)]
        Z = [sum(E[i], zero) for i in range(T)]
        P = [[E[i][j] / Z[i] for j in range(T)] for i in range(T)]
        Zs = Decimal(float(z))
        if keep is None:
            Pd = P
        else:
            Pd = [[Zs * P[i][j] if int(keep[i][j]) else zero for j in range(T)]
                  for i in range(T)]
        O = [[sum((Pd[i][j] * V[j][d] for j in range(T)), zero) for d in range(D)]
             for i in range(T)]
        LSE = [Z[i].ln() for i in range(T)]
        # dP = dO V^T over the full matrix.
        dP = [[sum((dO[i][d] * V[j][d] for d in range(D)), zero) for j in range(T)]
              for i in range(T)]
        if keep is not None:
            dP = [[Zs * dP[i][j] if int(keep[i][j]) else zero for j in range(T)]
                  for i in range(T)]
        # dS_i = J_i dP_i with J_i = diag(P_i) - P_i P_i^T.
        dS = []
        for i in range(T):
            row = []
            for j in range(T):
                acc = zero
                for kk in range(T):
                    jac = (P[i][j] if j == kk else zero) - P[i][j] * P[i][kk]
                    acc += jac * dP[i][kk]
                row.append(acc)
            dS.append(row)
        dV = [[sum((Pd[i][j] * dO[i][d] for i in range(T)), zero) for d in range(D)]
              for j in range(T)]
        dQ = [[s * sum((dS[i][j] * K[j][d] for j in range(T)), zero) for d in range(D)]
              for i in range(T)]
        dK = [[s * sum((dS[i][j] * Q[i][d] for i in range(T)), zero) for d in range(D)]
              for j in range(T)]
        to_f = lambda m: [[float(x) for x in r] for r in m]
        return {"O": to_f(O), "LSE": [float(x) for x in LSE], "dQ": to_f(dQ),
                "dK": to_f(dK), "dV": to_f(dV), "P": to_f(P)}
