"""fp64 oracle of the streaming chunk-causal softmax attention block -- TEST INFRASTRUCTURE.

Who may call this: see the package docstring (tests, smoke, the bench's CPU leg).

What it computes.  The SANA-WM Stage-1 DiT mixes softmax attention blocks into
its Gated DeltaNet stack (SGLang-diffusion cookbook page "SANA-WM", table
"Architecture & components", row "Attention"; the WorldFoundry guide's method
overview: alternating GDN and softmax attention blocks).  In streaming mode the
video is generated block by block with chunk-causal context (the cookbook's
serving-mode table, row "Batch streaming"), a rolling KV cache of the last
``num_cached_blocks`` blocks and ``sink_size`` sink frames (section
"Configuration reference": num_frame_per_block 3, num_cached_blocks 2,
sink_size 1).

Readings taken where the pages are silent:
  * Context of block n: the union of the frames of blocks max(0, n - C) .. n
    (C = cached blocks, the current block included) and the first S frames of
    the stream (the sink); every frame enters once, so a sink frame that is
    still inside a cached block is not counted twice.  All queries of block n
    see the whole context (chunk-causal: causal between blocks, full inside
    one).
  * Scores are q . k / sqrt(d) and the softmax runs over the context keys;
    no bias, no mask inside the context.  q and k are used as given
    (positional encodings and norms belong to the projections around the op).
"""
from __future__ import annotations

import numpy as np


def context_frames(block: int, frames_per_block: int, cached_blocks: int, sink_frames: int) -> list:
    """Frame indices (ascending, each once) that block `block` attends to."""
    if block < 0 or frames_per_block < 1 or cached_blocks < 0 or sink_frames < 0:
        raise ValueError("bad stream geometry")
    first = max(0, block - cached_blocks) * frames_per_block
    last = (block + 1) * frames_per_block  # exclusive
    frames = set(range(first, last))
    frames.update(f for f in range(sink_frames) if f < last)
    return sorted(frames)


def softmax_weights(q: np.ndarray, k: np.ndarray, scale: float | None = None) -> np.ndarray:
    """softmax(q k^T * scale) for one head: q [Lq, d], k [Lk, d] -> [Lq, Lk], fp64.

    The row maximum is subtracted before exponentiating (the softmax is
    unchanged by it; it only keeps exp() finite)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    s = (q @ k.T) * scale
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    return w


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None) -> np.ndarray:
    """softmax(q k^T * scale) v for one head: q [Lq, d], k [Lk, d], v [Lk, dv], fp64."""
    return softmax_weights(q, k, scale) @ np.asarray(v, np.float64)


def stream_block(q: np.ndarray, k_hist: np.ndarray, v_hist: np.ndarray, block: int, frame_tokens: int,
                 frames_per_block: int, cached_blocks: int, sink_frames: int) -> np.ndarray:
    """Output of block `block` for all (batch, head) pairs.

    q: [B, L_b, H, d] queries of the block; k_hist, v_hist: [B, >= (block+1) L_b, H, d]
    keys and values of every frame so far (frame-major tokens, the current
    block's last).  Returns o [B, L_b, H, d] in fp64."""
    lb = frames_per_block * frame_tokens
    frames = context_frames(block, frames_per_block, cached_blocks, sink_frames)
    rows = np.concatenate([np.arange(f * frame_tokens, (f + 1) * frame_tokens) for f in frames])
    B, L, H, d = q.shape
    if L != lb:
        raise ValueError("q must hold one block")
    o = np.zeros((B, L, H, v_hist.shape[-1]), np.float64)
    for b in range(B):
        for h in range(H):
            o[b, :, h] = attention(q[b, :, h], k_hist[b, rows, h], v_hist[b, rows, h])
    return o
