"""Seeded synthetic inputs for the frame-wise GDN forward.

This module is the only code that both the HIP path's tests and the CPU oracle
use.  It holds none of the method's arithmetic: it draws random numbers, lays
out shapes and rounds to bf16, nothing else.

Shapes come from the pages:
  * "SANA-WM" cookbook page, table "Architecture & components": the Stage-1
    DiT has 20 heads of head_dim 112 (hidden 2240) and an LTX-2 VAE with
    (T, H, W) strides (8, 32, 32); output is up to 704 x 1280 at 16 fps.
    A 704 x 1280 frame is therefore 22 x 40 = 880 latent tokens, and F pixel
    frames (F = 8k + 1, section "Configuration reference") are (F - 1)/8 + 1
    latent frames.
  * The same page's batch-streaming section generates 3 latent frames per
    block, so a streaming call carries 3 x 880 = 2,640 tokens.
Distributions (the workloads' recipe): q, k, v ~ N(0, 1); beta logits ~ N(0, 1);
one log-decay -softplus(z + 2), z ~ N(0, 1), per (frame, head) on the frame's
first token and 0 on every other token; an optional initial state ~ N(0, s^2).
Random numbers come from numpy's PCG64 ``default_rng(seed)``; per batch row the
draw order is q, k, v ([T, H, d] each), beta logits ([T, H]), gate z
([frames, H]); the initial state ([B, H, d, d]) is drawn last.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEADS = 20
HEAD_DIM = 112
LATENT_STRIDE_T, LATENT_STRIDE_HW = 8, 32
FRAME_H, FRAME_W = 704, 1280


def tokens_per_frame(height: int = FRAME_H, width: int = FRAME_W) -> int:
    """Latent tokens of one frame after the (32, 32) spatial VAE stride."""
    if height % LATENT_STRIDE_HW or width % LATENT_STRIDE_HW:
        raise ValueError("frame size must be a multiple of the VAE stride")
    return (height // LATENT_STRIDE_HW) * (width // LATENT_STRIDE_HW)


def latent_frames(pixel_frames: int) -> int:
    """Latent frames of an 8k+1 pixel clip under the temporal stride 8."""
    if pixel_frames < 1 or (pixel_frames - 1) % LATENT_STRIDE_T:
        raise ValueError("pixel frame count must be 8k + 1")
    return (pixel_frames - 1) // LATENT_STRIDE_T + 1


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    frames: int
    frame_tokens: int
    dtype: str            # "f32", "bf16" or "fp8" (E4M3FN): dtype of q, k, v
    seed: int
    calls: int = 1        # streaming: the sequence is split into this many equal calls
    state_std: float = 0.0  # > 0: initial state ~ N(0, state_std^2)
    head_dim: int = HEAD_DIM
    note: str = field(default="", compare=False)

    @property
    def seq_len(self) -> int:
        return self.frames * self.frame_tokens

    @property
    def tokens_per_call(self) -> int:
        assert self.seq_len % self.calls == 0
        return self.seq_len // self.calls


WORKLOADS = {
    w.name: w for w in (
        Workload("tiny_fp32", 1, 4, 4, 80, "f32", 101,
                 note="4 latent frames of 8x10 tokens, fp32"),
        Workload("window_2f", 1, HEADS, latent_frames(9), tokens_per_frame(), "bf16", 102,
                 note="9 pixel frames = 2 latent frames x 880 tokens"),
        Workload("clip_241f", 1, HEADS, latent_frames(241), tokens_per_frame(), "bf16", 103,
                 note="241 pixel frames = 31 latent frames x 880 = 27,280 tokens"),
        Workload("stream_3f_x10", 1, HEADS, 30, tokens_per_frame(), "bf16", 104, calls=10,
                 state_std=0.02, note="10 calls of 3 latent frames (2,640 tokens), state carried"),
        Workload("minute_cfg", 2, HEADS, latent_frames(961), tokens_per_frame(), "bf16", 105,
                 note="guidance pair, 961 pixel frames = 121 latent frames = 106,480 tokens"),
        Workload("window_2f_fp8", 1, HEADS, latent_frames(9), tokens_per_frame(), "fp8", 106,
                 note="9 pixel frames = 2 latent frames x 880 tokens, E4M3FN q/k/v"),
        Workload("clip_241f_fp8", 1, HEADS, latent_frames(241), tokens_per_frame(), "fp8", 107,
                 note="241 pixel frames = 31 latent frames x 880 = 27,280 tokens, E4M3FN q/k/v"),
    )
}


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    xf = np.ascontiguousarray(x, np.float32)
    b = xf.view(np.uint32)
    # no uint32 overflow: the largest non-NaN pattern 0xFF800000 plus 0x8000 fits
    out = ((b + (((b >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    nan = np.isnan(xf)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Values of x rounded to bf16 (RNE), returned as fp32."""
    return bf16_bits_to_f32(round_bf16_bits(x))


# OCP 8-bit floating point, E4M3FN ("OFP8" specification): 1 sign bit, 4
# exponent bits (bias 7), 3 mantissa bits; subnormals at exponent 0; no
# infinities; S.1111.111 is NaN; the largest finite magnitude is 448.
def _e4m3_magnitudes() -> np.ndarray:
    """The 127 non-negative finite E4M3FN values, indexed by code 0x00 .. 0x7E."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7))


def e4m3_codes_to_f32(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3FN codes (uint8) to fp32."""
    codes = np.asarray(codes, np.uint8)
    mag = np.append(_e4m3_magnitudes(), np.nan)[codes & 0x7F]
    return np.where(codes & 0x80, -mag, mag).astype(np.float32)


def round_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """fp32 -> E4M3FN codes: round to nearest, ties to even (on the mantissa's
    last bit), saturating at +-448; NaN -> 0x7F."""
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), 448.0)
    with np.errstate(divide="ignore"):
        e = np.clip(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6, 8)
    quantum = 2.0 ** (e - 3)
    qa = np.minimum(np.round(a / quantum) * quantum, 448.0)  # np.round: half to even
    codes = np.searchsorted(_e4m3_magnitudes(), qa).astype(np.uint8)
    codes = np.where(np.signbit(x), codes | 0x80, codes).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), codes).astype(np.uint8)


def _softplus(x):
    return np.logaddexp(0.0, x)


@dataclass
class Inputs:
    """q, k, v as fp32 arrays holding exactly the values the GPU receives
    (bf16- or E4M3FN-representable); ``*_bits`` hold the bf16 patterns (uint16)
    or the E4M3FN codes (uint8)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    state0: np.ndarray | None
    dtype: str
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None


def make_inputs(w: Workload, *, seed: int | None = None, seq_len: int | None = None,
                frame_tokens: int | None = None) -> Inputs:
    """Draw the workload's inputs.  ``seq_len`` / ``frame_tokens`` override the
    sizes (for reduced test cases, including ragged lengths)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    ft = frame_tokens or w.frame_tokens
    T = w.seq_len if seq_len is None else seq_len
    frames = -(-T // ft) if T else 0
    B, H, d = w.batch, w.heads, w.head_dim
    q = np.empty((B, T, H, d), np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q)
    beta = np.empty((B, T, H), np.float32)
    g = np.zeros((B, T, H), np.float32)
    for b in range(B):
        q[b] = rng.standard_normal((T, H, d), dtype=np.float32)
        k[b] = rng.standard_normal((T, H, d), dtype=np.float32)
        v[b] = rng.standard_normal((T, H, d), dtype=np.float32)
        beta[b] = rng.standard_normal((T, H), dtype=np.float32)
        z = rng.standard_normal((frames, H), dtype=np.float32).astype(np.float64)
        g[b, 0:T:ft] = (-_softplus(z + 2.0)).astype(np.float32)
    state0 = None
    if w.state_std > 0:
        state0 = (rng.standard_normal((B, H, d, d), dtype=np.float32) * np.float32(w.state_std))
    inp = Inputs(q, k, v, g, beta, state0, w.dtype)
    if w.dtype == "bf16":
        inp.q_bits, inp.k_bits, inp.v_bits = (round_bf16_bits(a) for a in (q, k, v))
        inp.q, inp.k, inp.v = (bf16_bits_to_f32(bb) for bb in (inp.q_bits, inp.k_bits, inp.v_bits))
    elif w.dtype == "fp8":
        # E4M3FN codes in *_bits (uint8)
        inp.q_bits, inp.k_bits, inp.v_bits = (round_e4m3_codes(a) for a in (q, k, v))
        inp.q, inp.k, inp.v = (e4m3_codes_to_f32(bb) for bb in (inp.q_bits, inp.k_bits, inp.v_bits))
    return inp


@dataclass
class AttnStream:
    """q, k, v of a whole stream of attention blocks: [B, blocks * L_b, H, d]
    bf16 patterns (``*_bits``) and their fp32 values."""
    q_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    block_tokens: int


def make_attn_stream(B: int, H: int, frame_tokens: int, frames_per_block: int, blocks: int, seed: int,
                     d: int = HEAD_DIM) -> AttnStream:
    """Seeded inputs of the streaming attention block: q, k, v ~ N(0, 1), drawn
    per batch row in the order q, k, v ([T, H, d] each), rounded to bf16."""
    rng = np.random.default_rng(seed)
    T = blocks * frames_per_block * frame_tokens
    arrs = [np.empty((B, T, H, d), np.float32) for _ in range(3)]
    for b in range(B):
        for a in arrs:
            a[b] = rng.standard_normal((T, H, d), dtype=np.float32)
    bits = [round_bf16_bits(a) for a in arrs]
    vals = [bf16_bits_to_f32(x) for x in bits]
    return AttnStream(*bits, *vals, block_tokens=frames_per_block * frame_tokens)


@dataclass
class LayerInputs:
    """x [B, T, H*112] and the layer's weights w_in [3 H 112 + 2 H, H 112],
    w_out [H 112, H 112] ([out, in] order): bf16 patterns (``*_bits``) and
    their fp32 values."""
    x_bits: np.ndarray
    w_in_bits: np.ndarray
    w_out_bits: np.ndarray
    x: np.ndarray
    w_in: np.ndarray
    w_out: np.ndarray
    heads: int
    frame_tokens: int


def make_layer_inputs(B: int, T: int, H: int, frame_tokens: int, seed: int) -> LayerInputs:
    """Seeded synthetic layer inputs: x ~ N(0, 1), weights ~ N(0, 1 / (H 112))
    (so every projected value is ~N(0, 1)), drawn in the order x, w_in, w_out
    and rounded to bf16.  Synthetic: no trained weights exist here."""
    rng = np.random.default_rng(seed)
    HD = H * HEAD_DIM
    x = rng.standard_normal((B, T, HD), dtype=np.float32)
    w_in = rng.standard_normal((3 * HD + 2 * H, HD), dtype=np.float32) * np.float32(1.0 / np.sqrt(HD))
    w_out = rng.standard_normal((HD, HD), dtype=np.float32) * np.float32(1.0 / np.sqrt(HD))
    bits = [round_bf16_bits(a) for a in (x, w_in, w_out)]
    vals = [bf16_bits_to_f32(b) for b in bits]
    return LayerInputs(*bits, *vals, heads=H, frame_tokens=frame_tokens)
