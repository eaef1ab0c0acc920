"""Exact rational brute force of the gated delta rule (test infrastructure only).

This is a second, deliberately different formulation of the same recurrence,
used to pin the fp64 oracle on tiny inputs.  Where the fp64 oracle works row by
row (decay, read, correct, write), this one builds each token's explicit
``d_k x d_k`` transition matrix and multiplies matrices in ``fractions.Fraction``
arithmetic:

    A_t = Diag(alpha_t) (I - beta_t k_t k_t^T)          (d_k x d_k)
    S_t = S_{t-1} A_t + beta_t v_t k_t^T                 (d_v x d_k)
    o_t = S_t q_t

That is the formula as stated for the method (decay matrix to the left of the
erase projector); the "FG2-GDN" page, section 5 ("Linear Attention as Recurrent
Memory") names the family of updates S_t = A_t S_{t-1} + write term in the
transposed orientation.  alpha is given directly as a rational (no logarithm);
with a scalar gate every channel gets the same alpha.

All arguments are nested Python lists of Fractions (or ints).
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence

Mat = List[List[Fraction]]


def _zeros(r: int, c: int) -> Mat:
    return [[Fraction(0)] * c for _ in range(r)]


def _matmul(a: Mat, b: Mat) -> Mat:
    n, m, p = len(a), len(b), len(b[0])
    out = _zeros(n, p)
    for i in range(n):
        for j in range(p):
            s = Fraction(0)
            for l in range(m):
                s += a[i][l] * b[l][j]
            out[i][j] = s
    return out


def transition(alpha: Sequence[Fraction], beta: Fraction, k: Sequence[Fraction]) -> Mat:
    """Diag(alpha) (I - beta k k^T) as an explicit d_k x d_k matrix."""
    dk = len(k)
    proj = [[(Fraction(1) if i == j else Fraction(0)) - beta * k[i] * k[j]
             for j in range(dk)] for i in range(dk)]
    diag = [[alpha[i] if i == j else Fraction(0) for j in range(dk)] for i in range(dk)]
    return _matmul(diag, proj)


def run(q, k, v, alpha, beta, S0=None):
    """Whole sequence for ONE head.

    q, k: T lists of d_k; v: T lists of d_v; alpha: T lists of d_k (channel gate;
    repeat the scalar for a scalar gate); beta: T values; S0: d_v x d_k or None.
    Returns (o: T lists of d_v, S_T: d_v x d_k), all Fractions.
    """
    T = len(q)
    dk = len(k[0])
    dv = len(v[0])
    S = _zeros(dv, dk) if S0 is None else [[Fraction(x) for x in row] for row in S0]
    outs = []
    for t in range(T):
        kt = [Fraction(x) for x in k[t]]
        A = transition([Fraction(a) for a in alpha[t]], Fraction(beta[t]), kt)
        S = _matmul(S, A)
        b = Fraction(beta[t])
        for i in range(dv):
            for c in range(dk):
                S[i][c] += b * Fraction(v[t][i]) * kt[c]
        outs.append([sum((S[i][c] * Fraction(q[t][c]) for c in range(dk)), Fraction(0))
                     for i in range(dv)])
    return outs, S


def run_fg2(q, k, v, alpha, sk, sv, S0=None):
    """Channel-wise write rates (FG2), whole sequence for ONE head, exactly.

    ``sk`` (T lists of d_k) and ``sv`` (T lists of d_v) are the square roots of
    the write rates beta^k and beta^v, given as rationals so that the scaled key
    k~ = sk * k and value v~ = sv * v stay rational.  Per token the explicit
    transition Diag(alpha_t) (I - k~ k~^T) multiplies the state and the write
    v~ k~^T is added ("FG2-GDN" page, sections 3.2 and 3.6: the tied
    diagonal-plus-rank-1 transition on the scaled keys).
    """
    T = len(q)
    dk = len(k[0])
    dv = len(v[0])
    S = _zeros(dv, dk) if S0 is None else [[Fraction(x) for x in row] for row in S0]
    outs = []
    for t in range(T):
        kt = [Fraction(sk[t][c]) * Fraction(k[t][c]) for c in range(dk)]
        vt = [Fraction(sv[t][i]) * Fraction(v[t][i]) for i in range(dv)]
        S = _matmul(S, transition([Fraction(a) for a in alpha[t]], Fraction(1), kt))
        for i in range(dv):
            for c in range(dk):
                S[i][c] += vt[i] * kt[c]
        outs.append([sum((S[i][c] * Fraction(q[t][c]) for c in range(dk)), Fraction(0))
                     for i in range(dv)])
    return outs, S


def run_gdn2(q, k, v, alpha, erase, write, S0=None):
    """Decoupled erase and write gates (Gated DeltaNet-2 reading), ONE head,
    exactly: per token the explicit transition Diag(alpha) (I - k (b*k)^T)
    multiplies the state and the write (w*v) k^T is added.  ``erase`` is T lists
    of d_k, ``write`` T lists of d_v."""
    T = len(q)
    dk = len(k[0])
    dv = len(v[0])
    S = _zeros(dv, dk) if S0 is None else [[Fraction(x) for x in row] for row in S0]
    outs = []
    for t in range(T):
        kt = [Fraction(x) for x in k[t]]
        et = [Fraction(erase[t][c]) * kt[c] for c in range(dk)]
        proj = [[(Fraction(1) if i == j else Fraction(0)) - kt[i] * et[j] for j in range(dk)]
                for i in range(dk)]
        diag = [[Fraction(alpha[t][i]) if i == j else Fraction(0) for j in range(dk)]
                for i in range(dk)]
        S = _matmul(S, _matmul(diag, proj))
        for i in range(dv):
            u = Fraction(write[t][i]) * Fraction(v[t][i])
            for c in range(dk):
                S[i][c] += u * kt[c]
        outs.append([sum((S[i][c] * Fraction(q[t][c]) for c in range(dk)), Fraction(0))
                     for i in range(dv)])
    return outs, S
