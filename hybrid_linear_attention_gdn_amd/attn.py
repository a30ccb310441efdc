"""Python binding of the streaming attention block (include/sanawm_attn.h).

Argument marshalling only: staging the block into the KV cache and the
attention itself run in the HIP kernels behind ``attn_block_fwd``.  There is
no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L
from .gdn import GdnError

HEAD_DIM = 112


def problem(B: int, H: int, frame_tokens: int, frames_per_block: int = 3, cached_blocks: int = 2,
            sink_frames: int = 1, o_dtype: torch.dtype = torch.float32) -> L.AttnProblem:
    """Stream geometry; the defaults are the SANA-WM streaming configuration."""
    code = {torch.float32: L.GDN_F32, torch.bfloat16: L.GDN_BF16}.get(o_dtype)
    if code is None:
        raise TypeError(f"unsupported output dtype {o_dtype}")
    return L.AttnProblem(B, H, HEAD_DIM, frame_tokens, frames_per_block, cached_blocks, sink_frames, code)


def _check(status: int):
    if status != L.GDN_OK:
        raise GdnError(status, L.load().gdn_last_error().decode())


def cache_bytes(p: L.AttnProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(L.load().attn_cache_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def new_cache(p: L.AttnProblem, device="cuda") -> torch.Tensor:
    """A KV cache for `p` (uninitialised: blocks fill it in order)."""
    return torch.empty(max(cache_bytes(p), 1), dtype=torch.uint8, device=device)


def block_fwd(p: L.AttnProblem, block: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cache: torch.Tensor,
              o: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Stage block `block`'s k, v into `cache` and return its attention output."""
    L_b = p.frame_tokens * p.frames_per_block
    shape = (p.batch, L_b, p.num_heads, HEAD_DIM)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if tuple(t.shape) != shape or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 GPU tensor of shape {shape}")
    if not cache.is_cuda or cache.dtype != torch.uint8 or not cache.is_contiguous():
        raise ValueError("cache must be a contiguous uint8 GPU tensor (see new_cache)")
    o_dtype = torch.float32 if p.o_dtype == L.GDN_F32 else torch.bfloat16
    if o is None:
        o = torch.empty(shape, dtype=o_dtype, device=q.device)
    elif tuple(o.shape) != shape or o.dtype != o_dtype or not o.is_cuda or not o.is_contiguous():
        raise ValueError(f"o must be a contiguous {o_dtype} GPU tensor of shape {shape}")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _check(L.load().attn_block_fwd(ctypes.byref(p), int(block), ctypes.c_void_p(q.data_ptr()),
                                   ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                   ctypes.c_void_p(cache.data_ptr()), cache.numel(), ctypes.c_void_p(o.data_ptr()),
                                   ctypes.c_void_p(stream.cuda_stream)))
    return o
