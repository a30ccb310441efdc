"""Pins of the CPU oracle to things other than itself (CPU only).

Each test names what fixes the expected value: a hand-worked example, exact
rational arithmetic, a closed form of the gated delta rule, a limit, or an
invariant.  The rule itself is the published gated delta rule named by the
"SANA-WM" cookbook page ("Architecture & components", row "Attention").
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle.chunked import gdn_chunked
from oracle.exact import gdn_exact
from oracle.recurrence import gdn_recurrence

RNG = np.random.default_rng(7)


def _rand(B, T, H, d, dv=None, *, gate_every=None, seed=0):
    r = np.random.default_rng(seed)
    dv = dv or d
    q = r.standard_normal((B, T, H, d))
    k = r.standard_normal((B, T, H, d))
    v = r.standard_normal((B, T, H, dv))
    beta = r.standard_normal((B, T, H))
    g = -np.logaddexp(0, r.standard_normal((B, T, H)) + 2)
    if gate_every:
        mask = (np.arange(T) % gate_every) == 0
        g = g * mask[None, :, None]
    return q, k, v, g, beta


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------- worked / exact

def test_hand_worked_example(golden_dir):
    """d = 2, two tokens, worked by hand (tests/golden/hand_d2.json)."""
    gd = json.load(open(os.path.join(golden_dir, "hand_d2.json")))
    sh = lambda a: np.array(a, np.float64)[None, :, None, :]  # noqa: E731
    g = np.log(np.array(gd["alpha"]))[None, :, None]
    beta = np.array(gd["beta"])[None, :, None]
    o, st = gdn_recurrence(sh(gd["q"]), sh(gd["k"]), sh(gd["v"]), g, beta,
                           beta_is_prob=True, qk_prenormalized=True)
    np.testing.assert_allclose(o[0, :, 0], np.array(gd["o"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(st[0, 0], np.array(gd["state"]), rtol=0, atol=1e-15)
    # the same example with raw (unnormalised) key/query lengths and beta as a logit:
    # sigmoid(0) = 1/2 and sigmoid(+inf) = 1
    scale = np.array([3.0, 5.0])[None, :, None, None]
    o2, st2 = gdn_recurrence(sh(gd["q"]) * 7.0, sh(gd["k"]) * scale, sh(gd["v"]), g,
                             np.array([0.0, np.inf])[None, :, None])
    np.testing.assert_allclose(o2[0, :, 0], np.array(gd["o"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(st2[0, 0], np.array(gd["state"]), rtol=0, atol=1e-15)


def _golden_exact(golden_dir):
    gd = json.load(open(os.path.join(golden_dir, "exact_d4.json")))
    fr = lambda rows: [[Fraction(x) for x in r] for r in rows]  # noqa: E731
    return gd, fr


def test_exact_rational_golden(golden_dir):
    """C oracle vs the stored exact-rational result (written by make_golden.py)."""
    gd, fr = _golden_exact(golden_dir)
    arr = lambda rows: np.array([[float(x) for x in r] for r in fr(rows)])  # noqa: E731
    q, k, v = (arr(gd[n])[None, :, None, :] for n in ("q", "k", "v"))
    alpha = np.array([float(Fraction(a)) for a in gd["alpha"]])
    beta = np.array([float(Fraction(b)) for b in gd["beta"]])
    S0 = arr(gd["state0"])[None, None]
    o, st = gdn_recurrence(q, k, v, np.log(alpha)[None, :, None], beta[None, :, None], S0,
                           beta_is_prob=True, qk_prenormalized=True)
    np.testing.assert_allclose(o[0, :, 0], arr(gd["o"]), rtol=0, atol=2e-15)
    np.testing.assert_allclose(st[0, 0], arr(gd["state"]), rtol=0, atol=2e-15)
    # the golden file itself must still be what the brute force gives
    outs, S = gdn_exact(fr(gd["q"]), fr(gd["k"]), fr(gd["v"]), [Fraction(a) for a in gd["alpha"]],
                        [Fraction(b) for b in gd["beta"]], fr(gd["state0"]))
    assert [[str(x) for x in r] for r in outs] == gd["o"]
    assert [[str(x) for x in r] for r in S] == gd["state"]


def test_exact_random_rational_cases():
    """Random rational cases with unit keys built from Pythagorean triples."""
    r = np.random.default_rng(11)
    triples = [(3, 4, 5), (5, 12, 13), (8, 15, 17), (7, 24, 25), (20, 21, 29)]
    for _ in range(5):
        T, d = 5, 3
        def unit():
            a, b, c = triples[r.integers(len(triples))]
            s = [Fraction(a, c) * (-1 if r.random() < .5 else 1), Fraction(b, c), Fraction(0)]
            perm = r.permutation(d)
            return [s[p] for p in perm]
        ks = [unit() for _ in range(T)]
        qs = [unit() for _ in range(T)]
        vs = [[Fraction(int(r.integers(-9, 10)), int(r.integers(1, 6))) for _ in range(d)] for _ in range(T)]
        al = [Fraction(int(r.integers(1, 11)), 10) for _ in range(T)]
        be = [Fraction(int(r.integers(0, 9)), 8) for _ in range(T)]
        S0 = [[Fraction(int(r.integers(-3, 4)), 4) for _ in range(d)] for _ in range(d)]
        outs, S = gdn_exact(qs, ks, vs, al, be, S0)
        f = lambda rows: np.array([[float(x) for x in row] for row in rows])  # noqa: E731
        o, st = gdn_recurrence(f(qs)[None, :, None], f(ks)[None, :, None], f(vs)[None, :, None],
                               np.log([float(a) for a in al])[None, :, None],
                               np.array([float(b) for b in be])[None, :, None], f(S0)[None, None],
                               beta_is_prob=True, qk_prenormalized=True)
        np.testing.assert_allclose(o[0, :, 0], f(outs), rtol=0, atol=1e-13)
        np.testing.assert_allclose(st[0, 0], f(S), rtol=0, atol=1e-13)
        oc, stc = gdn_chunked(f(qs)[None, :, None], f(ks)[None, :, None], f(vs)[None, :, None],
                              np.log([float(a) for a in al])[None, :, None],
                              np.array([float(b) for b in be])[None, :, None], f(S0)[None, None],
                              chunk=2, beta_is_prob=True, qk_prenormalized=True)
        np.testing.assert_allclose(oc[0, :, 0], f(outs), rtol=0, atol=1e-13)
        np.testing.assert_allclose(stc[0, 0], f(S), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- closed forms

def test_single_token_closed_form():
    """Zero state, one token: o = beta * v * (k_hat . q_hat) -- inclusive read-out, no scale."""
    q, k, v, g, beta = _rand(2, 1, 3, 112, seed=1)
    o, st = gdn_recurrence(q, k, v, g, beta)
    b = 1 / (1 + np.exp(-beta))
    kq = np.sum(_unit(k) * _unit(q), -1)
    np.testing.assert_allclose(o, (b * kq)[..., None] * v, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(st, np.einsum("bh,bhi,bhj->bhij", b[:, 0], v[:, 0], _unit(k)[:, 0]),
                               rtol=1e-12, atol=1e-15)


def test_beta_zero_decay_only():
    """beta = 0: nothing is written; o_t = exp(G_t) S0 q_hat_t, G_t the global cumulative log-decay."""
    q, k, v, g, _ = _rand(1, 50, 2, 16, gate_every=7, seed=2)
    S0 = np.random.default_rng(3).standard_normal((1, 2, 16, 16))
    o, st = gdn_recurrence(q, k, v, g, np.full(g.shape, -np.inf), S0)
    G = np.cumsum(g, axis=1)
    ref = np.exp(G)[..., None] * np.einsum("bhij,bthj->bthi", S0, _unit(q))
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(st, np.exp(G[:, -1])[..., None, None] * S0, rtol=1e-12)
    o0, st0 = gdn_recurrence(q, k, v, g, np.full(g.shape, -np.inf))
    assert not o0.any() and not st0.any()


def test_orthonormal_retrieval_exact():
    """alpha = 1, beta = 1, distinct standard-basis keys: reading a stored key returns its value."""
    d, T = 16, 10
    r = np.random.default_rng(4)
    keys = np.eye(d)[r.permutation(d)[:T]]
    v = r.standard_normal((1, T, 1, d))
    k = keys[None, :, None]
    q = np.concatenate([k[:, :1]] * T, axis=1)  # every step queries key 0
    o, st = gdn_recurrence(q, k, v, np.zeros((1, T, 1)), np.full((1, T, 1), np.inf))
    assert np.array_equal(o[0, :, 0], np.repeat(v[0, :1, 0], T, axis=0))
    # the final state maps each stored key to its value, bitwise
    assert np.array_equal(np.einsum("ij,tj->ti", st[0, 0], keys), v[0, :, 0])


def test_orthonormal_retrieval_random_basis_and_overwrite():
    d, T = 32, 20
    r = np.random.default_rng(5)
    Qm, _ = np.linalg.qr(r.standard_normal((d, d)))
    keys = Qm[:, :T].T
    v = r.standard_normal((T, d))
    o, st = gdn_recurrence(keys[None, :, None], keys[None, :, None], v[None, :, None],
                           np.zeros((1, T, 1)), np.full((1, T, 1), np.inf))
    np.testing.assert_allclose(np.einsum("ij,tj->ti", st[0, 0], keys), v, atol=2e-14)
    np.testing.assert_allclose(o[0, :, 0], v, atol=2e-14)  # o_t = S_t k_t = v_t
    # overwrite: writing key 0 again replaces its value
    k2 = np.concatenate([keys, keys[:1]])[None, :, None]
    v2 = np.concatenate([v, v[:1] * -3.0])[None, :, None]
    o2, st2 = gdn_recurrence(k2, k2, v2, np.zeros((1, T + 1, 1)), np.full((1, T + 1, 1), np.inf))
    np.testing.assert_allclose(st2[0, 0] @ keys[0], -3.0 * v[0], atol=2e-14)
    np.testing.assert_allclose(st2[0, 0] @ keys[1], v[1], atol=2e-14)


def test_small_beta_linear_attention_limit():
    """beta = eps -> 0: o -> (L o Gamma o Q K^T) diag(beta) V with error O(eps^2)."""
    q, k, v, g, _ = _rand(1, 40, 1, 8, gate_every=5, seed=6)
    qn, kn = _unit(q[0, :, 0]), _unit(k[0, :, 0])
    G = np.cumsum(g[0, :, 0])
    L = np.tril(np.ones((40, 40), bool))
    Gam = np.where(L, np.exp(np.where(L, G[:, None] - G[None, :], 0)), 0)
    errs = []
    for eps in (1e-2, 1e-3):
        o, _ = gdn_recurrence(q, k, v, g, np.full(g.shape, eps), beta_is_prob=True)
        lin = (Gam * (qn @ kn.T)) @ (eps * v[0, :, 0])
        errs.append(np.max(np.abs(o[0, :, 0] - lin)) / eps)  # relative to the O(eps) output
    assert errs[0] < 0.5  # the next term is O(eps)
    ratio = errs[0] / errs[1]
    assert 8.0 < ratio < 12.5, ratio  # relative error shrinks linearly: absolute error is O(eps^2)


# ---------------------------------------------------------------- chunked algebra

@pytest.mark.parametrize("chunk", [1, 16, 64, 80, 250])
def test_chunked_equals_recurrence(chunk):
    q, k, v, g, beta = _rand(1, 250, 2, 24, 20, gate_every=40, seed=8)
    S0 = 0.1 * np.random.default_rng(9).standard_normal((1, 2, 20, 24))
    o_r, s_r = gdn_recurrence(q, k, v, g, beta, S0)
    o_c, s_c = gdn_chunked(q, k, v, g, beta, S0, chunk=chunk)
    scale = np.sqrt(np.mean(o_r ** 2))
    assert np.max(np.abs(o_c - o_r)) <= 1e-13 * scale
    assert np.max(np.abs(s_c - s_r)) <= 1e-13 * np.sqrt(np.mean(s_r ** 2))


def test_chunked_floor_on_log_decay():
    """g = -inf (a full reset) stays finite in the chunked form through the -80 floor."""
    q, k, v, g, beta = _rand(1, 96, 1, 8, seed=10)
    g[0, 37, 0] = -np.inf
    o_r, s_r = gdn_recurrence(q, k, v, g, beta)
    o_c, s_c = gdn_chunked(q, k, v, g, beta, chunk=32)
    assert np.isfinite(o_c).all()
    np.testing.assert_allclose(o_c, o_r, rtol=0, atol=1e-13)
    np.testing.assert_allclose(s_c, s_r, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- streaming / invariants

def test_stream_split_equals_one_pass_bitwise():
    q, k, v, g, beta = _rand(1, 300, 3, 16, gate_every=30, seed=12)
    S0 = 0.02 * np.random.default_rng(13).standard_normal((1, 3, 16, 16))
    o1, s1 = gdn_recurrence(q, k, v, g, beta, S0)
    state, outs = S0, []
    cuts = [0, 90, 170, 171, 300]
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, state = gdn_recurrence(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], state)
        outs.append(o)
    assert np.array_equal(np.concatenate(outs, 1), o1)
    assert np.array_equal(state, s1)


def test_state_norm_contraction_bound():
    """||S_t||_F <= alpha_t ||S_{t-1}||_F + beta_t ||v_t||: I - beta k k^T is a contraction."""
    q, k, v, g, beta = _rand(1, 60, 1, 12, gate_every=6, seed=14)
    S = 0.5 * np.random.default_rng(15).standard_normal((1, 1, 12, 12))
    b = 1 / (1 + np.exp(-beta))
    for t in range(60):
        sl = slice(t, t + 1)
        _, S_new = gdn_recurrence(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], S)
        bound = np.exp(g[0, t, 0]) * np.linalg.norm(S) + b[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert np.linalg.norm(S_new) <= bound * (1 + 1e-12)
        S = S_new


def test_joint_linearity_in_values_and_state():
    q, k, v, g, beta = _rand(1, 70, 2, 10, gate_every=9, seed=16)
    r = np.random.default_rng(17)
    v2 = r.standard_normal(v.shape)
    S1, S2 = r.standard_normal((2, 1, 2, 10, 10))
    a, c = 0.7, -1.3
    o1, s1 = gdn_recurrence(q, k, v, g, beta, S1)
    o2, s2 = gdn_recurrence(q, k, v2, g, beta, S2)
    o3, s3 = gdn_recurrence(q, k, a * v + c * v2, g, beta, a * S1 + c * S2)
    np.testing.assert_allclose(o3, a * o1 + c * o2, atol=1e-12)
    np.testing.assert_allclose(s3, a * s1 + c * s2, atol=1e-12)


def test_head_and_batch_permutation_equivariance_and_threads():
    q, k, v, g, beta = _rand(2, 40, 5, 8, gate_every=8, seed=18)
    o, s = gdn_recurrence(q, k, v, g, beta, nthreads=1)
    o8, s8 = gdn_recurrence(q, k, v, g, beta, nthreads=8)
    assert np.array_equal(o, o8) and np.array_equal(s, s8)
    p = np.array([3, 0, 4, 1, 2])
    op, sp = gdn_recurrence(q[:, :, p], k[:, :, p], v[:, :, p], g[:, :, p], beta[:, :, p])
    assert np.array_equal(op, o[:, :, p]) and np.array_equal(sp, s[:, p])
    ob, sb = gdn_recurrence(q[::-1], k[::-1], v[::-1], g[::-1], beta[::-1])
    assert np.array_equal(ob, o[::-1]) and np.array_equal(sb, s[::-1])


def test_degenerate_inputs():
    q, k, v, g, beta = _rand(1, 20, 1, 8, seed=19)
    # zero key and query vectors normalise to zero: no write, no read
    k0 = k.copy(); k0[0, 5] = 0  # noqa: E702
    q0 = q.copy(); q0[0, 6] = 0  # noqa: E702
    o, _ = gdn_recurrence(q0, k0, v, g, beta)
    assert not o[0, 6].any()
    o_ref, s_ref = gdn_recurrence(q0, k0, v, g, beta)
    assert np.isfinite(o).all()
    # g = -inf wipes the state: the output after it equals a fresh run from that token
    g2 = g.copy(); g2[0, 10] = -np.inf  # noqa: E702
    o2, _ = gdn_recurrence(q, k, v, g2, beta)
    g_fresh = g[:, 10:].copy(); g_fresh[0, 0] = 0.0  # noqa: E702  (decay of a zero state is moot)
    o_fresh, _ = gdn_recurrence(q[:, 10:], k[:, 10:], v[:, 10:], g_fresh, beta[:, 10:])
    np.testing.assert_allclose(o2[:, 10:], o_fresh, atol=1e-14)
    # empty sequence: the state passes through unchanged
    S0 = np.random.default_rng(20).standard_normal((1, 1, 8, 8))
    oe, se = gdn_recurrence(q[:, :0], k[:, :0], v[:, :0], g[:, :0], beta[:, :0], S0)
    assert oe.shape == (1, 0, 1, 8) and np.array_equal(se, S0)
    # beta logits of +-inf give exactly 1 and 0
    o_inf, _ = gdn_recurrence(q[:, :1], k[:, :1], v[:, :1], g[:, :1], np.full((1, 1, 1), np.inf))
    o_one, _ = gdn_recurrence(q[:, :1], k[:, :1], v[:, :1], g[:, :1], np.ones((1, 1, 1)), beta_is_prob=True)
    assert np.array_equal(o_inf, o_one)
    assert math.isfinite(float(o_ref.sum())) and np.isfinite(s_ref).all()
