"""fp64 oracle of the bidirectional (dense) frame-wise Gated DeltaNet -- TEST INFRASTRUCTURE.

Who may call this: see the package docstring (tests, smoke, the bench's CPU leg).

What it computes.  The SGLang-diffusion cookbook page "SANA-WM" describes a
dense checkpoint that generates a whole clip in one shot with full
bidirectional context instead of chunk-causal context (serving-mode table, row
"Dense bidirectional"; section "Dense bidirectional"), while its DiT's token
mixer is the frame-wise Gated DeltaNet (table "Architecture & components").
The pages do not say how the recurrent mixer becomes bidirectional.  Readings
taken:

  * Reverse scan: the gated delta rule of ``recurrence`` run over the tokens
    in reverse order.  Its decays sit on the same frame boundaries as the
    forward scan's: the forward scan applies alpha_t when it moves from token
    t - 1 to token t, so the reverse scan applies alpha_{t+1} when it moves
    from token t + 1 to token t, and nothing when it enters the last token.
    With frame-wise gates (g non-zero only on a frame's first token) a
    token's contribution to another then decays by the gates of the frame
    starts between them, whichever side it lies on.
  * The reverse scan's entry state (the context after the last token) is
    ``state_in`` (zero by default) and its exit state is the state after
    token 0.
  * Combination: o_t = o_t(forward) + o_t(reverse), each scan including
    token t's own write.
"""
from __future__ import annotations

import numpy as np

from oracle.recurrence import gdn_recurrence


def successor_decays(g: np.ndarray) -> np.ndarray:
    """[B, T, H] log-decays the reverse scan applies at each token: token t
    takes token t + 1's, the last token none."""
    g = np.asarray(g, np.float64)
    out = np.zeros_like(g)
    out[:, :-1] = g[:, 1:]
    return out


def reverse_scan(q, k, v, g, beta, state_in=None, **kw):
    """The reverse scan in the original token order: (o [B, T, H, dv], exit state or None)."""
    rev = lambda a: np.ascontiguousarray(np.asarray(a)[:, ::-1])  # noqa: E731
    o, st = gdn_recurrence(rev(q), rev(k), rev(v), rev(successor_decays(g)), rev(beta), state_in, **kw)
    return np.ascontiguousarray(o[:, ::-1]), st


def bidirectional(q, k, v, g, beta, **kw):
    """o_forward + o_reverse, both scans from a zero state."""
    kw = dict(kw, want_state=False)
    o_f, _ = gdn_recurrence(q, k, v, g, beta, None, **kw)
    o_r, _ = reverse_scan(q, k, v, g, beta, None, **kw)
    return o_f + o_r
