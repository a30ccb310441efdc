"""Python binding of the layer around the scan (include/sanawm_gdn.h, "The layer
around the scan"): ``in_proj``, ``out_proj`` and ``layer_fwd``.

Argument marshalling only: the projections and the scan run in the HIP
kernels behind the C ABI.  Weights are bf16 in [out, in] order:
w_in [3 H 112 + 2 H, H 112], w_out [H 112, H 112]."""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L
from .gdn import GdnError, _check, _dtype_code

HEAD_DIM = 112


def problem(B, T, H, frame_tokens, y_dtype=torch.float32, bidirectional=False) -> L.LayerProblem:
    return L.LayerProblem(B, T, H, frame_tokens, _dtype_code(y_dtype),
                          L.GDN_LAYER_BIDIRECTIONAL if bidirectional else 0)


def workspace_bytes(p: L.LayerProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(L.load().gdn_layer_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(name, t, shape, dtype):
    if t is None or tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor of shape {tuple(shape)}")


def _stream(t, stream):
    return ctypes.c_void_p((stream or torch.cuda.current_stream(t.device)).cuda_stream)


def in_proj(x, w_in, frame_tokens, *, stream=None):
    """x [B, T, H*112] bf16 -> (q, k, v [B, T, H, 112] bf16, beta, g [B, T, H] fp32)."""
    B, T, HD = x.shape
    H = HD // HEAD_DIM
    _need("x", x, (B, T, H * HEAD_DIM), torch.bfloat16)
    _need("w_in", w_in, (3 * HD + 2 * H, HD), torch.bfloat16)
    q, k, v = (torch.empty((B, T, H, HEAD_DIM), dtype=torch.bfloat16, device=x.device) for _ in range(3))
    beta, g = (torch.empty((B, T, H), dtype=torch.float32, device=x.device) for _ in range(2))
    p = problem(B, T, H, frame_tokens)
    _check(L.load().gdn_in_proj(ctypes.byref(p), _ptr(x), _ptr(w_in), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                _ptr(g), _stream(x, stream)))
    return q, k, v, beta, g


def out_proj(o, w_out, *, y_dtype=torch.float32, stream=None):
    """o [B, T, H*112] (or [B, T, H, 112]) bf16 -> y [B, T, H*112]."""
    if o.dim() not in (3, 4):
        raise ValueError("o must be [B, T, H*112] or [B, T, H, 112]")
    B, T = o.shape[:2]
    HD = o.shape[2] * (o.shape[3] if o.dim() == 4 else 1)
    _need("o", o, o.shape, torch.bfloat16)
    _need("w_out", w_out, (HD, HD), torch.bfloat16)
    y = torch.empty((B, T, HD), dtype=y_dtype, device=o.device)
    p = problem(B, T, HD // HEAD_DIM, 1, y_dtype)
    _check(L.load().gdn_out_proj(ctypes.byref(p), _ptr(o), _ptr(w_out), _ptr(y), _stream(o, stream)))
    return y


def layer_fwd(x, w_in, w_out, frame_tokens, state_in=None, state_out=None, *, y_dtype=torch.float32,
              bidirectional=False, workspace=None, stream=None):
    """The whole layer: y = out_proj(scan(in_proj(x))).  Returns (y, state_out)."""
    B, T, HD = x.shape
    H = HD // HEAD_DIM
    _need("x", x, (B, T, H * HEAD_DIM), torch.bfloat16)
    _need("w_in", w_in, (3 * HD + 2 * H, HD), torch.bfloat16)
    _need("w_out", w_out, (HD, HD), torch.bfloat16)
    for name, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None:
            _need(name, t, (B, H, HEAD_DIM, HEAD_DIM), torch.float32)
    y = torch.empty((B, T, HD), dtype=y_dtype, device=x.device)
    p = problem(B, T, H, frame_tokens, y_dtype, bidirectional)
    need = workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(L.load().gdn_layer_fwd(ctypes.byref(p), _ptr(x), _ptr(w_in), _ptr(w_out), _ptr(state_in),
                                  _ptr(state_out), _ptr(y), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                  _stream(x, stream)))
    return y, state_out


__all__ = ["problem", "workspace_bytes", "in_proj", "out_proj", "layer_fwd", "GdnError"]
