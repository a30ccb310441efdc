"""The chunk algebra the MFMA kernels implement, checked in fp64 against the
token-by-token oracle (CPU only).

The intra-chunk step writes, per chunk of n tokens, a record of K~, Q', P''
and M and the scales; the state pass then runs, with S the d_v x d_k state:

    A_ri = beta_r rk_r rk_i e^(G_r - G_i) (k_r . k_i)    (i < r),   T = (I + A)^-1
    P_ri = rq_r rk_i e^(G_r - G_i) (q_r . k_i)          (i <= r),  P' = P T
    M    = K^T diag(rk_i e^(G_n - G_i)) T
    K~   = -diag(beta gamma rk) K,   Q' = diag(gamma rq) Q + P' K~,   P'' = P' diag(beta)
    R    = diag(beta) V + K~ S^T,    S^T <- gamma_n S^T + M R
    O    = Q' S^T + P'' V            (= diag(gamma rq) Q S^T + P' R)

with raw (unnormalised) K, Q, V rows, rk = 1/|k|, rq = 1/|q|, G the chunk's
inclusive cumulative log-decay (floored at -80) and gamma = e^G.  This is a
rearrangement of the gated delta rule (the rule named by the "SANA-WM"
cookbook page, "Architecture & components", row "Attention"); the test fixes
that the rearrangement is exact, so that the GPU kernels' only departures
from the oracle are their roundings.
"""
import numpy as np
import pytest

from oracle.recurrence import gdn_recurrence


def _chunk_form(q, k, v, g, beta, state_in, C):
    """fp64 evaluation of the kernels' chunk algebra for one (b, h)."""
    T, dk = k.shape
    S = np.array(state_in, np.float64)           # [dv, dk]
    o = np.zeros((T, v.shape[1]))
    bt = 1.0 / (1.0 + np.exp(-beta))
    rk = 1.0 / np.linalg.norm(k, axis=1)
    rq = 1.0 / np.linalg.norm(q, axis=1)
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        K, Q, V = k[sl], q[sl], v[sl]
        n = K.shape[0]
        G = np.cumsum(np.maximum(g[sl], -80.0))
        gam = np.exp(G)
        b, r_k, r_q = bt[sl], rk[sl], rq[sl]
        dec = np.exp(G[:, None] - G[None, :])
        strict = np.tril(np.ones((n, n), bool), -1)
        incl = np.tril(np.ones((n, n), bool))
        A = np.where(strict, b[:, None] * r_k[:, None] * r_k[None, :] * dec * (K @ K.T), 0.0)
        Tm = np.linalg.inv(np.eye(n) + A)
        P = np.where(incl, r_q[:, None] * r_k[None, :] * dec * (Q @ K.T), 0.0)
        Pp = P @ Tm
        M = K.T @ ((r_k * np.exp(G[-1] - G))[:, None] * Tm)
        Kt = -(b * gam * r_k)[:, None] * K
        Qp = (gam * r_q)[:, None] * Q + Pp @ Kt
        Ppp = Pp * b[None, :]
        St = S.T                                    # [dk, dv]
        R = b[:, None] * V + Kt @ St
        o[sl] = Qp @ St + Ppp @ V
        # the textbook output form gives the same rows
        assert np.allclose(o[sl], (gam * r_q)[:, None] * (Q @ St) + Pp @ R, rtol=0, atol=1e-12 * (1 + np.abs(o[sl]).max()))
        S = (gam[-1] * St + M @ R).T
    return o, S


@pytest.mark.parametrize("T,C,d", [(173, 80, 112), (64, 16, 12), (81, 80, 20)])
def test_chunk_algebra_equals_recurrence(T, C, d):
    r = np.random.default_rng(11 + T)
    B, H = 1, 2
    q = r.standard_normal((B, T, H, d))
    k = r.standard_normal((B, T, H, d))
    v = r.standard_normal((B, T, H, d))
    beta = r.standard_normal((B, T, H))
    # frame-wise gates: one log-decay every 40 tokens, 0 elsewhere
    g = -np.logaddexp(0, r.standard_normal((B, T, H)) + 2) * ((np.arange(T) % 40) == 0)[None, :, None]
    s0 = 0.02 * r.standard_normal((B, H, d, d))
    o_ref, s_ref = gdn_recurrence(q, k, v, g, beta, s0)
    for h in range(H):
        o, s = _chunk_form(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h], beta[0, :, h], s0[0, h], C)
        scale = np.sqrt(np.mean(o_ref[0, :, h] ** 2))
        assert np.max(np.abs(o - o_ref[0, :, h])) <= 1e-12 * scale
        assert np.max(np.abs(s - s_ref[0, h])) <= 1e-12 * np.sqrt(np.mean(s_ref[0, h] ** 2))


def test_chunk_algebra_records_have_the_stated_shapes():
    # M is d_k x n and P' lower triangular n x n: what the intra-chunk step stores
    r = np.random.default_rng(3)
    n, d = 80, 112
    K, Q = r.standard_normal((n, d)), r.standard_normal((n, d))
    rk, rq = 1 / np.linalg.norm(K, axis=1), 1 / np.linalg.norm(Q, axis=1)
    b = 1 / (1 + np.exp(-r.standard_normal(n)))
    G = np.zeros(n)
    dec = np.exp(G[:, None] - G[None, :])
    A = np.tril(b[:, None] * rk[:, None] * rk[None, :] * dec * (K @ K.T), -1)
    Tm = np.linalg.inv(np.eye(n) + A)
    assert np.allclose(np.triu(Tm, 1), 0.0)            # T lower triangular, unit diagonal
    assert np.allclose(np.diag(Tm), 1.0)
    Pp = np.tril(rq[:, None] * rk[None, :] * dec * (Q @ K.T)) @ Tm
    assert np.allclose(np.triu(Pp, 1), 0.0)
    M = K.T @ (rk[:, None] * Tm)
    assert M.shape == (d, n)
