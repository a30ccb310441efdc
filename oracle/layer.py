"""fp64 oracle of the GDN layer with its projections -- TEST INFRASTRUCTURE.

Who may call this: see the package docstring (tests, smoke, the bench's CPU leg).

What it computes.  The SGLang-diffusion cookbook page "SANA-WM" (table
"Architecture & components") gives the DiT's width (hidden 2240 = 20 heads x
112) and names its token mixer, the frame-wise Gated DeltaNet; it prints no
projection.  Readings taken (plain linear maps without biases, weights in
[out, in] order):

    [q | k | v | b | a] = x W_in^T          W_in: [3 H d + 2 H, H d]
    beta = b                                (logits; the scan applies the sigmoid)
    g_t  = -softplus(a_t) if t is a frame's first token (t % frame_tokens == 0),
           0 otherwise                      (one log-decay per frame and head)
    o    = the scan over (q, k, v, g, beta) (``recurrence``, or ``bidirectional``)
    y    = o W_out^T                        W_out: [H d, H d]

The DiT runs in bf16 (the diffusers "SANA-WM" page loads its checkpoints as
torch.bfloat16), so q, k, v and o are bf16 tensors between the steps: with
``bf16_intermediates`` (the default) they are rounded to bf16 (nearest, ties
to even) where the model stores them.  Everything else is fp64 on the values
given.
"""
from __future__ import annotations

import numpy as np

from oracle.bidirectional import bidirectional
from oracle.recurrence import gdn_recurrence

D = 112


def round_bf16(x):
    """x rounded to the nearest bfloat16 (8 significant bits, ties to even),
    as float64; straight from fp64, without an fp32 step."""
    m, e = np.frexp(np.asarray(x, np.float64))  # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0), e - 8)


def softplus(x):
    """log(1 + e^x) without overflow."""
    return np.logaddexp(0.0, x)


def in_proj(x, w_in, H, frame_tokens):
    """x [B, T, H d] -> q, k, v [B, T, H, d], beta, g [B, T, H]."""
    x = np.asarray(x, np.float64)
    B, T, HD = x.shape
    assert HD == H * D and w_in.shape == (3 * HD + 2 * H, HD)
    z = x @ np.asarray(w_in, np.float64).T
    q, k, v = (z[..., i * HD:(i + 1) * HD].reshape(B, T, H, D) for i in range(3))
    beta = z[..., 3 * HD:3 * HD + H]
    a = z[..., 3 * HD + H:]
    first = (np.arange(T) % frame_tokens == 0)[None, :, None]
    g = np.where(first, -softplus(a), 0.0)
    return q, k, v, beta, g


def layer(x, w_in, w_out, H, frame_tokens, state_in=None, *, bidirectional_scan=False, bf16_intermediates=True):
    """(y [B, T, H d], exit state or None)."""
    q, k, v, beta, g = in_proj(x, w_in, H, frame_tokens)
    if bf16_intermediates:
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    B, T = q.shape[:2]
    if bidirectional_scan:
        o, st = bidirectional(q, k, v, g, beta), None
    else:
        o, st = gdn_recurrence(q, k, v, g, beta, state_in)
    if bf16_intermediates:
        o = round_bf16(o)
    y = o.reshape(B, T, H * D) @ np.asarray(w_out, np.float64).T
    return y, st
