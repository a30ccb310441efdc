"""ctypes front-end of the plain fp64 C recurrence (``gdn_recurrence.c``).

TEST INFRASTRUCTURE: see the package docstring for who may call this.

The recurrence is the published gated delta rule that the SGLang-diffusion
cookbook page "SANA-WM" (table "Architecture & components", row "Attention")
names as the frame-wise Gated DeltaNet; the C file's header states it and the
readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_recurrence.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_gdn.so")

BETA_IS_PROB = 1
QK_PRENORMALIZED = 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_gdn_fwd.restype = ctypes.c_int
        lib.oracle_gdn_fwd.argtypes = [ctypes.c_int] * 5 + [dp] * 8 + [ctypes.c_uint, ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def default_threads(units: int) -> int:
    return max(1, min(units, os.cpu_count() or 1))


def gdn_recurrence(q, k, v, g, beta, state_in=None, *, beta_is_prob=False,
                   qk_prenormalized=False, nthreads=None, want_state=True):
    """fp64 token-by-token GDN forward.

    q, k: [B, T, H, dk]; v: [B, T, H, dv]; g (log-decay), beta (logits, or
    probabilities with ``beta_is_prob``): [B, T, H]; state_in: [B, H, dv, dk]
    or None (zero state).  Inputs are widened to fp64 exactly.
    Returns (o [B, T, H, dv], state_out [B, H, dv, dk] or None).
    """
    q, k, v, g, beta, state_in = map(_f64, (q, k, v, g, beta, state_in))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, T, H, dk) and v.shape == (B, T, H, dv)
    assert g.shape == (B, T, H) and beta.shape == (B, T, H)
    if state_in is not None:
        assert state_in.shape == (B, H, dv, dk)
    o = np.empty((B, T, H, dv), np.float64)
    st = np.empty((B, H, dv, dk), np.float64) if want_state else None
    flags = (BETA_IS_PROB if beta_is_prob else 0) | (QK_PRENORMALIZED if qk_prenormalized else 0)
    n = nthreads if nthreads else default_threads(B * H)
    rc = _load().oracle_gdn_fwd(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(state_in), _ptr(st), _ptr(o), flags, n)
    if rc != 0:
        raise ValueError("oracle_gdn_fwd rejected its arguments")
    return o, st
