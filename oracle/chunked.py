"""fp64 chunked (UT / WY) form of the gated delta rule -- TEST INFRASTRUCTURE.

Derived here from the token recurrence of ``gdn_recurrence.c`` (the published
gated delta rule of Yang, Kautz & Hatamizadeh, ICLR 2025, that the "SANA-WM"
cookbook page's "Architecture & components" table names as the frame-wise
Gated DeltaNet).  It is not the oracle of record -- the recurrence is -- but
it pins the chunk algebra the GPU path evaluates and hands out its per-chunk
intermediates.

Derivation, per (batch, head) and per chunk of n <= C consecutive tokens with
entry state S0 (d_v x d_k).  Write the recurrence as
    S_r = alpha_r S_{r-1} + u_r k_r^T,   u_r = beta_r (v_r - alpha_r S_{r-1} k_r)
(normalised k, q).  With G_r = sum_{j<=r} log alpha_j (chunk-local, inclusive)
and gamma_r = exp(G_r):
    S_r = gamma_r S0 + sum_{i<=r} exp(G_r - G_i) u_i k_i^T.
Substituting into u_r gives the unit-lower-triangular system
    (I + A) U = diag(beta) V - diag(beta * gamma) K S0^T,
    A_ri = beta_r exp(G_r - G_i) (k_r . k_i)   for i < r, 0 otherwise,
so with Tm = (I + A)^-1, W = Tm diag(beta*gamma) K and Ut = Tm diag(beta) V:
    U      = Ut - W S0^T
    O      = diag(gamma) Q S0^T + (L o Gamma o Q K^T) U        (L: i <= r)
    S_next = gamma_n S0 + U^T diag(exp(G_n - G_i)) K.
The log-decays are clamped at -80 before the cumulative sum so that the
differences G_r - G_i never meet (-inf) - (-inf); the clamp changes a decay
factor by at most exp(-80) and is the same reading the GPU path takes.
"""
from __future__ import annotations

import numpy as np

G_FLOOR = -80.0


def _normalize(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-6)


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def chunk_tensors(kc, vc, qc, bc, gc):
    """Per-chunk quantities that do not depend on the entry state.

    kc, qc: [n, dk] normalised; vc: [n, dv]; bc: [n] beta; gc: [n] log-decay.
    Returns a dict with G, gamma, A, Tm, W, Ut, Pm (= L o Gamma o Q K^T) and
    decay_to_end (= exp(G_n - G_i)).
    """
    n = kc.shape[0]
    G = np.cumsum(np.maximum(gc, G_FLOOR))
    diff = G[:, None] - G[None, :]
    incl = np.tril(np.ones((n, n), bool))
    strict = np.tril(np.ones((n, n), bool), -1)
    Gam = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)
    A = np.where(strict, bc[:, None] * Gam * (kc @ kc.T), 0.0)
    Tm = np.linalg.inv(np.eye(n) + A)
    gamma = np.exp(G)
    W = Tm @ ((bc * gamma)[:, None] * kc)
    Ut = Tm @ (bc[:, None] * vc)
    Pm = Gam * (qc @ kc.T)
    return dict(G=G, gamma=gamma, A=A, Tm=Tm, W=W, Ut=Ut, Pm=Pm,
                decay_to_end=np.exp(G[-1] - G) if n else G)


def gdn_chunked(q, k, v, g, beta, state_in=None, *, chunk=80, beta_is_prob=False,
                qk_prenormalized=False, keep=False):
    """Chunked fp64 GDN forward.  Shapes as in ``recurrence.gdn_recurrence``.

    Returns (o, state_out) or, with ``keep``, (o, state_out, per_unit) where
    per_unit[(b, h)] is a list of per-chunk dicts (chunk_tensors plus U, S0).
    """
    q, k, v, g, beta = (np.asarray(a, np.float64) for a in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    qn = q if qk_prenormalized else _normalize(q)
    kn = k if qk_prenormalized else _normalize(k)
    bt = beta if beta_is_prob else _sigmoid(beta)
    o = np.zeros((B, T, H, dv))
    st = np.zeros((B, H, dv, dk))
    kept = {}
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if state_in is None else np.array(state_in[b, h], np.float64)
            rec = []
            for c0 in range(0, T, chunk):
                sl = slice(c0, min(c0 + chunk, T))
                kc, qc, vc = kn[b, sl, h], qn[b, sl, h], v[b, sl, h]
                ct = chunk_tensors(kc, vc, qc, bt[b, sl, h], g[b, sl, h])
                U = ct["Ut"] - ct["W"] @ S.T
                o[b, sl, h] = ct["gamma"][:, None] * (qc @ S.T) + ct["Pm"] @ U
                if keep:
                    ct.update(U=U, S0=S.copy())
                    rec.append(ct)
                S = ct["gamma"][-1] * S + U.T @ (ct["decay_to_end"][:, None] * kc)
            st[b, h] = S
            if keep:
                kept[(b, h)] = rec
    return (o, st, kept) if keep else (o, st)
