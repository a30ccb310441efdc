"""Python binding of libsanawm_gdn: ``gdn_fwd``, ``gdn_chunk_step`` and ``gdn_bidir_fwd``.

Argument marshalling only.  Every step of the forward runs in the HIP
kernels behind the C ABI (include/sanawm_gdn.h); PyTorch provides the device
memory and the stream.  There is no CPU or PyTorch fallback: a missing
library or a non-GPU tensor raises.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        lib = L.load()
        super().__init__(f"{lib.gdn_status_string(status).decode()}: {message}")
        self.status = status


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return L.GDN_F32
    if t == torch.bfloat16:
        return L.GDN_BF16
    if t == torch.float8_e4m3fn:
        return L.GDN_FP8_E4M3
    raise TypeError(f"unsupported dtype {t} (float32, bfloat16 or float8_e4m3fn)")


def problem(B, T, H, dk, dv, qkv_dtype, o_dtype, *, beta_is_prob=False, qk_prenormalized=False,
            reverse=False) -> L.Problem:
    flags = ((L.GDN_FLAG_BETA_IS_PROB if beta_is_prob else 0) |
             (L.GDN_FLAG_QK_PRENORMALIZED if qk_prenormalized else 0) |
             (L.GDN_FLAG_REVERSE if reverse else 0))
    return L.Problem(B, T, H, dk, dv, _dtype_code(qkv_dtype), _dtype_code(o_dtype), flags)


def _check(status: int):
    if status != L.GDN_OK:
        raise GdnError(status, L.load().gdn_last_error().decode())


def workspace_bytes(p: L.Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(L.load().gdn_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def bidir_workspace_bytes(p: L.Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(L.load().gdn_bidir_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def workspace_layout(p: L.Problem) -> L.WorkspaceLayout:
    lay = L.WorkspaceLayout()
    _check(L.load().gdn_workspace_layout(ctypes.byref(p), ctypes.byref(lay)))
    return lay


def chunk_len() -> int:
    return L.load().gdn_chunk_len()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call(entry, q, k, v, g, beta, state_in, state_out, o, o_dtype, beta_is_prob, qk_prenormalized,
          workspace, stream, reverse=False, bidir=False, no_alloc=False):
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d_k]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    want = {"q": (q, (B, T, H, dk)), "k": (k, (B, T, H, dk)), "v": (v, (B, T, H, dv)), "g": (g, (B, T, H)),
            "beta": (beta, (B, T, H))}
    for name, (t, shape) in want.items():
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("g and beta must be float32")
    for name, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None and (tuple(t.shape) != (B, H, dv, dk) or t.dtype != torch.float32 or not t.is_cuda
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor of shape {(B, H, dv, dk)}")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=o_dtype, device=q.device)
    elif tuple(o.shape) != (B, T, H, dv) or not o.is_contiguous() or o.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("o must be a contiguous float32/bfloat16 tensor of shape [B, T, H, d_v]")
    p = problem(B, T, H, dk, dv, q.dtype, o.dtype, beta_is_prob=beta_is_prob,
                qk_prenormalized=qk_prenormalized, reverse=reverse)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    states = () if bidir else (_ptr(state_in), _ptr(state_out))
    if no_alloc:  # the library's own fixed workspace
        ws_args = ()
    else:
        need = bidir_workspace_bytes(p) if bidir else workspace_bytes(p)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        ws_args = (_ptr(workspace), ctypes.c_size_t(workspace.numel()))
    status = entry(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), *states,
                   _ptr(o), *ws_args, ctypes.c_void_p(stream.cuda_stream))
    _check(status)
    return o, state_out


def gdn_fwd(q, k, v, g, beta, state_in=None, state_out="new", o=None, *, o_dtype=torch.float32,
            beta_is_prob=False, qk_prenormalized=False, reverse=False, workspace=None, stream=None):
    """Frame-wise GDN forward over q, k [B,T,H,d_k], v [B,T,H,d_v] (bf16, fp8 E4M3FN or
    fp32), g (log-decay), beta (logits) [B,T,H] fp32.  ``state_out``: "new" allocates the
    final state, None skips it, a tensor receives it (may be ``state_in``).
    ``reverse``: the reverse scan (GDN_FLAG_REVERSE).  Returns (o, state_out)."""
    if isinstance(state_out, str):
        B, _, H, dk = q.shape
        state_out = torch.empty((B, H, v.shape[-1], dk), dtype=torch.float32, device=q.device)
    return _call(L.load().gdn_fwd, q, k, v, g, beta, state_in, state_out, o, o_dtype, beta_is_prob,
                 qk_prenormalized, workspace, stream, reverse=reverse)


def gdn_fwd_no_alloc(q, k, v, g, beta, state_in, state_out, o, *, beta_is_prob=False, qk_prenormalized=False,
                     reverse=False, stream=None):
    """gdn_fwd on the library's fixed per-device workspace (gdn_fwd_no_alloc):
    o and state_out (or None) are caller tensors; nothing is allocated."""
    return _call(L.load().gdn_fwd_no_alloc, q, k, v, g, beta, state_in, state_out, o, o.dtype, beta_is_prob,
                 qk_prenormalized, None, stream, reverse=reverse, no_alloc=True)


def gdn_bidir_fwd(q, k, v, g, beta, o=None, *, o_dtype=torch.float32, beta_is_prob=False,
                  qk_prenormalized=False, workspace=None, stream=None):
    """Bidirectional layer (gdn_bidir_fwd): the forward scan plus the reverse scan,
    both from a zero state.  Returns o."""
    o, _ = _call(L.load().gdn_bidir_fwd, q, k, v, g, beta, None, None, o, o_dtype, beta_is_prob,
                 qk_prenormalized, workspace, stream, bidir=True)
    return o


def gdn_chunk_step(q, k, v, g, beta, state_in, state_out="new", o=None, *, o_dtype=torch.float32,
                   beta_is_prob=False, qk_prenormalized=False, reverse=False, workspace=None, stream=None):
    """One streaming call: like gdn_fwd with state_in required and T a multiple of
    the chunk length (80), which makes a rollout bitwise equal to one pass."""
    if isinstance(state_out, str):
        B, _, H, dk = q.shape
        state_out = torch.empty((B, H, v.shape[-1], dk), dtype=torch.float32, device=q.device)
    return _call(L.load().gdn_chunk_step, q, k, v, g, beta, state_in, state_out, o, o_dtype, beta_is_prob,
                 qk_prenormalized, workspace, stream, reverse=reverse)
