"""Exact-rational brute force of the gated delta rule -- TEST INFRASTRUCTURE.

Evaluates the product form of the published gated delta rule (the update the
"SANA-WM" cookbook page's "Architecture & components" table names as the
frame-wise Gated DeltaNet) with explicit matrices over ``fractions.Fraction``:

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t.

No normalisation, sigmoid or exponential is applied: the caller passes unit
keys / queries with rational entries and rational alpha, beta, so the result
is exact.  Meant for d <= 4 and a handful of tokens.
"""
from __future__ import annotations

from fractions import Fraction


def _matmul(a, b):
    return [[sum((a[i][m] * b[m][j] for m in range(len(b))), Fraction(0))
             for j in range(len(b[0]))] for i in range(len(a))]


def gdn_exact(qs, ks, vs, alphas, betas, S0=None):
    """qs, ks: T lists of dk Fractions (unit norm); vs: T lists of dv Fractions;
    alphas, betas: T Fractions; S0: dv x dk list of lists or None.
    Returns (outputs: T lists of dv Fractions, final state dv x dk)."""
    dk, dv = len(ks[0]), len(vs[0])
    S = [[Fraction(0)] * dk for _ in range(dv)] if S0 is None else [list(map(Fraction, r)) for r in S0]
    outs = []
    for q, k, v, a, b in zip(qs, ks, vs, alphas, betas):
        # explicit I - beta k k^T
        M = [[(Fraction(1) if i == j else Fraction(0)) - b * k[i] * k[j] for j in range(dk)] for i in range(dk)]
        SM = _matmul(S, M)
        S = [[a * SM[i][j] + b * v[i] * k[j] for j in range(dk)] for i in range(dv)]
        outs.append([sum((S[i][j] * q[j] for j in range(dk)), Fraction(0)) for i in range(dv)])
    return outs, S
