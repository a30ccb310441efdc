"""Shared helpers of the GPU tests: upload seeded inputs, run the HIP path,
run the oracle on the same values, and measure the error the way the
parity bar is stated (max |o - o_ref| / rms(o_ref))."""
from __future__ import annotations

import numpy as np
import torch

from hybrid_linear_attention_gdn_amd.inputs import Inputs

# Parity bars: bf16 inputs with fp32 state, and the fp32 path.
TOL_BF16 = 1e-2
TOL_F32 = 1e-4


def to_device(inp: Inputs, dev="cuda", fp32=False):
    """Upload the inputs.  ``fp32``: q, k, v as fp32 tensors of the same values
    (a bf16 workload then runs on the fp32 vector-ALU kernels)."""
    if fp32:
        q, k, v = (torch.from_numpy(np.asarray(a, np.float32)).to(dev) for a in (inp.q, inp.k, inp.v))
    elif inp.dtype == "bf16":
        up = lambda bits: torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
        q, k, v = up(inp.q_bits), up(inp.k_bits), up(inp.v_bits)
    elif inp.dtype == "fp8":  # E4M3FN codes
        up8 = lambda codes: torch.from_numpy(codes).to(dev).view(torch.float8_e4m3fn)  # noqa: E731
        q, k, v = up8(inp.q_bits), up8(inp.k_bits), up8(inp.v_bits)
    else:
        q, k, v = (torch.from_numpy(a).to(dev) for a in (inp.q, inp.k, inp.v))
    g = torch.from_numpy(inp.g).to(dev)
    beta = torch.from_numpy(inp.beta).to(dev)
    s0 = None if inp.state0 is None else torch.from_numpy(inp.state0).to(dev)
    return q, k, v, g, beta, s0


def rel_max_err(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(x - ref)) / rms) if ref.size else 0.0


def state_err(st, ref) -> float:
    """Exit-state error: the largest over the (b, h) units of max|S - S_ref| /
    rms(S_ref) within the unit.  The tolerance the sources fix is on o; each
    unit's state is an independent result of its own scale (a head's state can
    be several times another's), so each is held to the bar against its own
    rms rather than the rms over all heads."""
    x = np.asarray(st, np.float64)
    r = np.asarray(ref, np.float64)
    assert x.shape == r.shape and x.ndim >= 2
    x, r = x.reshape(-1, *x.shape[-2:]), r.reshape(-1, *r.shape[-2:])
    worst = 0.0
    for u in range(x.shape[0]):
        rms = np.sqrt(np.mean(r[u] * r[u]))
        if rms > 0:
            worst = max(worst, float(np.max(np.abs(x[u] - r[u])) / rms))
        elif np.any(x[u] != 0):
            worst = float("inf")
    return worst


def oracle_for(inp: Inputs, heads=None, batches=None, t_end=None):
    """fp64 oracle on (a subset of) the same values the GPU receives."""
    from oracle.recurrence import gdn_recurrence
    sl = lambda a: a  # noqa: E731
    q, k, v, g, beta, s0 = inp.q, inp.k, inp.v, inp.g, inp.beta, inp.state0
    if t_end is not None:
        q, k, v, g, beta = (a[:, :t_end] for a in (q, k, v, g, beta))
    if batches is not None:
        q, k, v, g, beta = (a[batches] for a in (q, k, v, g, beta))
        s0 = None if s0 is None else s0[batches]
    if heads is not None:
        q, k, v, g, beta = (a[:, :, heads] for a in (q, k, v, g, beta))
        s0 = None if s0 is None else s0[:, heads]
    del sl
    return gdn_recurrence(q, k, v, g, beta, s0)
