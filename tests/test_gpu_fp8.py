"""FP8 (OCP E4M3FN) q, k, v on the MFMA path, fp32 state (the FP8 Stage-1
precision of the SGLang cookbook page "SANA-WM", section "Configuration
reference"), against the fp64 oracle on the decoded values.

Every E4M3FN value is exact in bf16 and the kernels widen the codes to bf16
as they load them, so the fp8 path must reproduce the bf16 path fed with the
same values bit for bit: that equality is checked at a ragged length with an
initial state, at B = 1 and B = 2 x 20 heads (40 units: 160 state-pass
workgroups beside the intra-chunk blocks) and in streaming.  The parity bar is the bf16 path's, 1e-2 of rms(o_ref)."""
import sys

import numpy as np
import pytest
import torch

from hybrid_linear_attention_gdn_amd import gdn
from hybrid_linear_attention_gdn_amd.inputs import WORKLOADS, Workload, make_inputs
from tests.helpers import TOL_BF16, oracle_for, rel_max_err, state_err, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check(o, st, o_ref, s_ref, label):
    eo, es = rel_max_err(o, o_ref), state_err(st, s_ref)
    _say(f"[{label}] max|o-o_ref|/rms = {eo:.3e}   state: {es:.3e}   (bar {TOL_BF16:g})")
    assert np.isfinite(o).all()
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


def _as_bf16(t):
    return t.float().to(torch.bfloat16)  # exact: every E4M3FN value is a bf16 value


def test_window_2f_fp8_config():
    w = WORKLOADS["window_2f_fp8"]
    _say("case window_2f_fp8")
    inp = make_inputs(w)
    q, k, v, g, beta, s0 = to_device(inp)
    assert q.dtype == torch.float8_e4m3fn
    o, st = gdn.gdn_fwd(q, k, v, g, beta, s0)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_for(inp)
    _check(o.cpu().numpy(), st.cpu().numpy(), o_ref, s_ref, "window_2f_fp8")


@pytest.mark.parametrize("T,B,H", [(1, 1, 2), (79, 1, 3), (81, 2, 2), (250, 1, 4)])
def test_fp8_ragged_and_small(T, B, H):
    w = Workload("ragged_fp8", B, H, 1, 10**9, "fp8", 50 + T, state_std=0.05)
    inp = make_inputs(w, seq_len=T, frame_tokens=97)
    _say("case fp8 ragged", T, B, H)
    q, k, v, g, beta, s0 = to_device(inp)
    o, st = gdn.gdn_fwd(q, k, v, g, beta, s0)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_for(inp)
    _check(o.cpu().numpy(), st.cpu().numpy(), o_ref, s_ref, f"fp8 ragged T={T}")


@pytest.mark.parametrize("B", [1, 2])
def test_fp8_equals_bf16_on_the_same_values(B):
    """B = 2: 40 (b, h) units, so the state pass takes 160 workgroups and the
    intra-chunk blocks share the rest of the GPU with it."""
    w = WORKLOADS["clip_241f_fp8"]
    inp = make_inputs(w, seq_len=5063)
    inp.state0 = (0.02 * np.random.default_rng(8).standard_normal((1, 20, 112, 112))).astype(np.float32)
    q, k, v, g, beta, s0 = to_device(inp)
    if B == 2:
        cat = lambda t: torch.cat([t, t], 0).contiguous()  # noqa: E731
        q, k, v, g, beta, s0 = (cat(t) for t in (q, k, v, g, beta, s0))
    _say("case fp8 == bf16, T=5063, B =", B)
    res = {}
    for o_dtype in (torch.float32, torch.bfloat16):
        o8, s8 = gdn.gdn_fwd(q, k, v, g, beta, s0, o_dtype=o_dtype)
        o16, s16 = gdn.gdn_fwd(_as_bf16(q), _as_bf16(k), _as_bf16(v), g, beta, s0, o_dtype=o_dtype)
        torch.cuda.synchronize()
        assert torch.equal(o8, o16) and torch.equal(s8, s16)
        res[o_dtype] = (o8, s8)
    o8, s8 = res[torch.float32]
    o_ref, s_ref = oracle_for(inp, heads=[0, 19], batches=[0])
    _check(o8.cpu().numpy()[:1][:, :, [0, 19]], s8.cpu().numpy()[:1][:, [0, 19]], o_ref, s_ref,
           f"fp8 T=5063 B={B}, heads 0, 19")


@pytest.mark.parametrize("reverse", [False, True])
def test_fp8_equals_bf16_full_shape_dense_gates(reverse):
    """The fp8 and bf16 instantiations of the kernels are scheduled
    differently, so bitwise equality of their results on the same values, at
    the full 27,280 x 20 shape with a gate on every token (every chunk then
    takes the decay and intra-chunk paths), in both directions and both o
    types, checks that neither schedule reads a value too early."""
    w = WORKLOADS["clip_241f_fp8"]
    inp = make_inputs(w, frame_tokens=1)
    q, k, v, g, beta, s0 = to_device(inp)
    _say(f"case fp8 == bf16, 27,280 x 20, dense gates, reverse={reverse}")
    for o_dtype in (torch.float32, torch.bfloat16):
        o8, s8 = gdn.gdn_fwd(q, k, v, g, beta, s0, o_dtype=o_dtype, reverse=reverse)
        o16, s16 = gdn.gdn_fwd(_as_bf16(q), _as_bf16(k), _as_bf16(v), g, beta, s0, o_dtype=o_dtype,
                               reverse=reverse)
        torch.cuda.synchronize()
        assert torch.isfinite(o8.float()).all()
        assert torch.equal(o8, o16) and torch.equal(s8, s16)


def test_fp8_streaming_rollout_equals_one_pass():
    w = WORKLOADS["clip_241f_fp8"]
    Tc, calls = 2640, 4
    inp = make_inputs(w, seq_len=Tc * calls)
    inp.state0 = (0.02 * np.random.default_rng(9).standard_normal((1, 20, 112, 112))).astype(np.float32)
    q, k, v, g, beta, s0 = to_device(inp)
    _say("case fp8 streaming: 4 chunk steps of 2,640 tokens")
    state = s0.clone()
    outs = []
    for c in range(calls):
        sl = slice(c * Tc, (c + 1) * Tc)
        o, state = gdn.gdn_chunk_step(q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous(),
                                      g[:, sl].contiguous(), beta[:, sl].contiguous(), state, state)
        outs.append(o)
    o_one, s_one = gdn.gdn_fwd(q, k, v, g, beta, s0)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, 1), o_one) and torch.equal(state, s_one)


def test_clip_241f_fp8_all_heads():
    """The full 27,280-token layer in fp8; the oracle checks all 20 heads."""
    w = WORKLOADS["clip_241f_fp8"]
    _say("case clip_241f_fp8 (27,280 tokens x 20 heads), all heads")
    inp = make_inputs(w)
    q, k, v, g, beta, s0 = to_device(inp)
    o, st = gdn.gdn_fwd(q, k, v, g, beta, s0)
    torch.cuda.synchronize()
    o, st = o.cpu().numpy(), st.cpu().numpy()
    assert np.isfinite(o).all()
    o_ref, s_ref = oracle_for(inp)
    _check(o, st, o_ref, s_ref, "clip_241f_fp8 all 20 heads")


def test_fp8_rejects_other_head_dims():
    # fp8 inputs run on the MFMA kernels only, which take d_k = d_v = 112
    q = torch.zeros(1, 80, 2, 64, dtype=torch.float8_e4m3fn, device="cuda")
    g = torch.zeros(1, 80, 2, device="cuda")
    with pytest.raises(gdn.GdnError):
        gdn.gdn_fwd(q, q, q, g, g)
