"""Pins of the bidirectional GDN oracle (oracle/bidirectional.py) to closed forms
and invariants that follow from the gated delta rule and the readings stated in
that module (reverse scan with the decays on the same frame boundaries; sum of
the two scans), not to the oracle itself."""
import numpy as np
import pytest

from oracle import bidirectional as BD
from oracle.recurrence import gdn_recurrence


def _frame_gates(rng, B, T, H, ft):
    g = np.zeros((B, T, H))
    g[:, 0:T:ft] = -rng.uniform(0.05, 1.5, size=(B, len(range(0, T, ft)), H))
    return g


def _orthonormal_case(rng, T, H, d, ft):
    """Keys: distinct standard basis vectors times positive factors (unit after
    normalisation), beta = 1: the delta rule then writes v_t k_t^T untouched."""
    k = np.zeros((1, T, H, d))
    for h in range(H):
        perm = rng.permutation(d)[:T]
        k[0, np.arange(T), h, perm] = rng.uniform(0.5, 2.0, size=T)
    q = rng.normal(size=(1, T, H, d))
    v = rng.normal(size=(1, T, H, 5))
    beta = np.ones((1, T, H))
    return q, k, v, _frame_gates(rng, 1, T, H, ft), beta


def test_closed_form_orthonormal_keys():
    # o_t = sum_s exp(Gc[max(s,t)] - Gc[min(s,t)]) (k^_s . q^_t) v_s  +  (k^_t . q^_t) v_t,
    # Gc the inclusive cumulative log-decay: the same boundary decays on both sides
    rng = np.random.default_rng(11)
    T, H, d, ft = 13, 2, 16, 3
    q, k, v, g, beta = _orthonormal_case(rng, T, H, d, ft)
    o = BD.bidirectional(q, k, v, g, beta, beta_is_prob=True)
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    for h in range(H):
        Gc = np.cumsum(g[0, :, h])
        dots = kn[0, :, h] @ qn[0, :, h].T  # [s, t]
        want = np.zeros((T, 5))
        for t in range(T):
            for s in range(T):
                w = np.exp(Gc[max(s, t)] - Gc[min(s, t)]) * dots[s, t]
                want[t] += w * v[0, s, h] * (2.0 if s == t else 1.0)
        np.testing.assert_allclose(o[0, :, h], want, rtol=0, atol=1e-12)


def test_reverse_scan_exit_state_closed_form():
    # an entry state in directions no key touches is only decayed: by all gates
    # after token 0 (the last token applies none); the writes decay to token 0
    rng = np.random.default_rng(12)
    T, H, d, ft = 10, 1, 16, 4
    q, k, v, g, beta = _orthonormal_case(rng, T, H, d, ft)
    used = np.flatnonzero(k[0, :, 0].any(axis=0))
    S0 = rng.normal(size=(1, H, 5, d))
    S0[..., used] = 0.0
    _, st = BD.reverse_scan(q, k, v, g, beta, S0, beta_is_prob=True)
    Gc = np.cumsum(g[0, :, 0])
    kn = k[0, :, 0] / np.linalg.norm(k[0, :, 0], axis=-1, keepdims=True)
    want = np.exp(Gc[-1] - Gc[0]) * S0[0, 0]
    for s in range(T):
        want += np.exp(Gc[s] - Gc[0]) * np.outer(v[0, s, 0], kn[s])
    np.testing.assert_allclose(st[0, 0], want, rtol=0, atol=1e-12)


def test_single_token_is_twice_the_forward():
    rng = np.random.default_rng(13)
    q, k, v = (rng.normal(size=(2, 1, 3, 8)) for _ in range(3))
    g, beta = rng.normal(size=(2, 1, 3)), rng.normal(size=(2, 1, 3))
    o_f, _ = gdn_recurrence(q, k, v, g, beta)
    np.testing.assert_allclose(BD.bidirectional(q, k, v, g, beta), 2 * o_f, rtol=0, atol=1e-15)


def test_zero_gate_cuts_both_directions():
    # alpha = 0 at a frame start: neither side sees across it
    rng = np.random.default_rng(14)
    B, T, H, d, ft, cut = 1, 24, 2, 8, 4, 12
    q, k, v = (rng.normal(size=(B, T, H, d)) for _ in range(3))
    beta = rng.normal(size=(B, T, H))
    g = _frame_gates(rng, B, T, H, ft)
    g[:, cut] = -1e4  # exp underflows to 0 in fp64
    o = BD.bidirectional(q, k, v, g, beta)
    pre = BD.bidirectional(q[:, :cut], k[:, :cut], v[:, :cut], g[:, :cut], beta[:, :cut])
    post = BD.bidirectional(q[:, cut:], k[:, cut:], v[:, cut:], g[:, cut:], beta[:, cut:])
    np.testing.assert_allclose(o[:, :cut], pre, rtol=0, atol=1e-13)
    np.testing.assert_allclose(o[:, cut:], post, rtol=0, atol=1e-13)


def test_mirrored_sequence_mirrors_the_output():
    # reversing the tokens and moving each gate with its frame boundary
    # (mirrored token j enters from j - 1 across the boundary of original
    # tokens T-1-j and T-j) reverses the bidirectional output
    rng = np.random.default_rng(15)
    B, T, H, d, ft = 2, 21, 2, 8, 5
    q, k, v = (rng.normal(size=(B, T, H, d)) for _ in range(3))
    beta = rng.normal(size=(B, T, H))
    g = _frame_gates(rng, B, T, H, ft)
    o = BD.bidirectional(q, k, v, g, beta)
    m = lambda a: a[:, ::-1].copy()  # noqa: E731
    gm = np.zeros_like(g)
    for j in range(1, T):
        gm[:, j] = g[:, T - j]
    gm[:, 0] = rng.normal(size=(B, H))  # acts on the zero entry state only
    om = BD.bidirectional(m(q), m(k), m(v), gm, m(beta))
    np.testing.assert_allclose(om, o[:, ::-1], rtol=0, atol=1e-12)


def test_successor_decays():
    g = np.arange(12, dtype=np.float64).reshape(1, 6, 2)
    s = BD.successor_decays(g)
    np.testing.assert_array_equal(s[0, :5], g[0, 1:])
    assert not s[0, 5].any()
