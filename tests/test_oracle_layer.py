"""Pins of the layer oracle (oracle/layer.py): the softplus gate's closed
values, where the gate lands, the row order of W_in and the orientation of
both weights, each against values fixed independently of the oracle."""
import math

import numpy as np

from oracle import layer as LY
from oracle.recurrence import gdn_recurrence

D = LY.D


def test_softplus_values():
    x = np.array([0.0, 1.0, -1.0, 50.0, -50.0, 800.0])
    want = [math.log(2.0), math.log(1.0 + math.e), math.log(1.0 + 1.0 / math.e), 50.0 + math.exp(-50.0),
            math.exp(-50.0), 800.0]
    np.testing.assert_allclose(LY.softplus(x), want, rtol=1e-15, atol=0)


def test_round_bf16_values():
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -9, -(2 - 2.0 ** -9), 3.0e-5, 0.0,
                  1 + 2.0 ** -8 + 2.0 ** -30])
    want = [1.0, 1.0, 1 + 2.0 ** -6, 1.0, -2.0, 3.0e-5, 0.0, 1 + 2.0 ** -7]
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even 1; 1 + 3 2^-8
    # halfway between 1 + 2^-7 and 1 + 2^-6 (even); just above a tie rounds up
    got = LY.round_bf16(x)
    np.testing.assert_array_equal(got[[0, 1, 2, 3, 4, 6, 7]], np.array(want)[[0, 1, 2, 3, 4, 6, 7]])
    assert abs(got[5] - 3.0e-5) <= 2.0 ** -8 * 3.0e-5  # within half a bf16 ulp (unit roundoff 2^-8)
    r = np.random.default_rng(0).normal(size=1000)
    assert (np.abs(LY.round_bf16(r) - r) <= 2.0 ** -8 * np.abs(r)).all()
    # exactly 8 significant bits: every result is a multiple of 2^(e - 7) for its binade 2^e
    m, e = np.frexp(LY.round_bf16(r))
    np.testing.assert_array_equal(m * 256, np.round(m * 256))


def _weights(rng, H):
    HD = H * D
    return rng.normal(size=(3 * HD + 2 * H, HD)) / math.sqrt(HD), rng.normal(size=(HD, HD)) / math.sqrt(HD)


def test_gate_only_on_frame_starts():
    rng = np.random.default_rng(1)
    H, T, ft = 2, 10, 4
    w_in, _ = _weights(rng, H)
    x = rng.normal(size=(1, T, H * D))
    _, _, _, beta, g = LY.in_proj(x, w_in, H, ft)
    a = x @ w_in[3 * H * D + H:].T  # the a rows: the last H of W_in
    for t in range(T):
        if t % ft == 0:
            np.testing.assert_allclose(g[0, t], -np.log1p(np.exp(a[0, t])), rtol=1e-13)
        else:
            assert not g[0, t].any()
    np.testing.assert_allclose(beta[0], x[0] @ w_in[3 * H * D:3 * H * D + H].T, rtol=1e-13)


def test_block_row_order_and_orientation():
    # W_in = [I; P; 2I; 0; c 1] (P a permutation), W_out = a non-symmetric matrix:
    # q = x, k = x P^T, v = 2x, beta = 0 (sigmoid 1/2), a = c sum(x); y = o W_out^T
    rng = np.random.default_rng(2)
    H, T, ft = 1, 7, 3
    HD = H * D
    perm = rng.permutation(HD)
    Pm = np.eye(HD)[perm]
    w_in = np.concatenate([np.eye(HD), Pm, 2 * np.eye(HD), np.zeros((H, HD)), 0.1 * np.ones((H, HD))])
    w_out = np.triu(rng.normal(size=(HD, HD)))
    x = rng.normal(size=(1, T, HD))
    y, st = LY.layer(x, w_in, w_out, H, ft, bf16_intermediates=False)
    q = x.reshape(1, T, H, D)
    k = x[..., perm].reshape(1, T, H, D)
    a = 0.1 * x.sum(-1, keepdims=True)
    g = np.where((np.arange(T) % ft == 0)[None, :, None], -np.logaddexp(0, a), 0.0)
    o, st2 = gdn_recurrence(q, k, 2 * q, g, np.zeros((1, T, H)))
    np.testing.assert_allclose(y, o.reshape(1, T, HD) @ w_out.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st, st2, rtol=1e-12, atol=1e-14)


def test_bidirectional_layer_uses_both_scans():
    rng = np.random.default_rng(3)
    H, T, ft = 1, 9, 3
    w_in, w_out = _weights(rng, H)
    x = rng.normal(size=(1, T, H * D))
    yb, none = LY.layer(x, w_in, w_out, H, ft, bidirectional_scan=True, bf16_intermediates=False)
    yf, _ = LY.layer(x, w_in, w_out, H, ft, bf16_intermediates=False)
    assert none is None
    # the last token's reverse scan sees only itself: y_b - y_f there is the
    # single-token write of the last token projected through W_out
    q, k, v, beta, g = LY.in_proj(x, w_in, H, ft)
    kn = k[0, -1, 0] / np.linalg.norm(k[0, -1, 0])
    qn = q[0, -1, 0] / np.linalg.norm(q[0, -1, 0])
    b = 1 / (1 + np.exp(-beta[0, -1, 0]))
    o_last = b * v[0, -1, 0] * (kn @ qn)
    np.testing.assert_allclose(yb[0, -1] - yf[0, -1], o_last @ w_out.T, rtol=1e-10, atol=1e-12)
