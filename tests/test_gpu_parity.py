"""Parity of the HIP path with the fp64 oracle (needs an MI355X).

Bars: max |o - o_ref| <= 1e-2 * rms(o_ref) for bf16 inputs with fp32 state,
<= 1e-4 * rms(o_ref) on the fp32 path; the final state against rms(state_ref)
with the same bars.  Inputs are the seeded synthetic workloads of
``hybrid_linear_attention_gdn_amd.inputs`` (shapes from the SANA-WM pages).
"""
import sys

import numpy as np
import pytest
import torch

from hybrid_linear_attention_gdn_amd import gdn
from hybrid_linear_attention_gdn_amd.inputs import WORKLOADS, make_inputs
from tests.helpers import TOL_BF16, TOL_F32, oracle_for, rel_max_err, state_err, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(inp, *, fp32=False, o_dtype=torch.float32, state=True):
    """fp32: upload q, k, v as fp32 (the vector-ALU kernels) instead of bf16 (the MFMA kernels)."""
    q, k, v, g, beta, s0 = to_device(inp, fp32=fp32)
    o, st = gdn.gdn_fwd(q, k, v, g, beta, s0, "new" if state else None, o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), (st.cpu().numpy() if st is not None else None)


def _check(inp, o, st, o_ref, s_ref, tol, label):
    eo = rel_max_err(o, o_ref)
    es = state_err(st, s_ref) if st is not None else 0.0
    _say(f"[{label}] max|o-o_ref|/rms = {eo:.3e}   state: {es:.3e}   (bar {tol:g})")
    assert np.isfinite(o).all()
    assert eo <= tol, eo
    assert es <= tol, es


def test_tiny_fp32_config():
    w = WORKLOADS["tiny_fp32"]
    _say("case tiny_fp32", w)
    inp = make_inputs(w)
    o, st = _run(inp)
    o_ref, s_ref = oracle_for(inp)
    _check(inp, o, st, o_ref, s_ref, TOL_F32, "tiny_fp32")


@pytest.mark.parametrize("fp32", [False, True])
def test_window_2f_config(fp32):
    w = WORKLOADS["window_2f"]
    _say("case window_2f fp32 inputs=", fp32)
    inp = make_inputs(w)
    o, st = _run(inp, fp32=fp32)
    o_ref, s_ref = oracle_for(inp)
    _check(inp, o, st, o_ref, s_ref, TOL_BF16, "window_2f")


@pytest.mark.parametrize("T,B,H", [(1, 1, 2), (79, 1, 3), (81, 2, 2), (250, 1, 4), (400, 2, 3)])
def test_ragged_and_small(T, B, H):
    from hybrid_linear_attention_gdn_amd.inputs import Workload
    w = Workload("ragged", B, H, 1, 10**9, "bf16", 7 + T, state_std=0.05)
    inp = make_inputs(w, seq_len=T, frame_tokens=97)
    _say("case ragged", T, B, H)
    for fp32 in (False, True):
        o, st = _run(inp, fp32=fp32)
        o_ref, s_ref = oracle_for(inp)
        _check(inp, o, st, o_ref, s_ref, TOL_BF16, f"ragged T={T} fp32 inputs={fp32}")


def test_portable_general_head_dims_fp32():
    from hybrid_linear_attention_gdn_amd.inputs import Workload
    w = Workload("dims", 2, 3, 3, 50, "f32", 31, state_std=0.1, head_dim=64)
    inp = make_inputs(w)
    inp.v = inp.v[..., :48].copy()
    inp.state0 = inp.state0[:, :, :48, :].copy()
    _say("case portable dk=64 dv=48")
    o, st = _run(inp)
    o_ref, s_ref = oracle_for(inp)
    _check(inp, o, st, o_ref, s_ref, TOL_F32, "dk64 dv48 fp32")


def test_portable_largest_and_smallest_head_dims_fp32():
    # d = 128 is the largest the portable kernels take (their LDS is sized for it); d = 1 the smallest
    from hybrid_linear_attention_gdn_amd.inputs import Workload
    for d, frame_tokens in ((128, 85), (1, 45)):  # T = 170 and 90: ragged last chunks
        w = Workload(f"d{d}", 1, 2, 2, frame_tokens, "f32", 33 + d, state_std=0.1, head_dim=d)
        T = w.seq_len
        inp = make_inputs(w)
        _say(f"case portable dk=dv={d} T={T}")
        o, st = _run(inp)
        o_ref, s_ref = oracle_for(inp)
        _check(inp, o, st, o_ref, s_ref, TOL_F32, f"d{d} fp32")


def test_clip_241f_full_config():
    w = WORKLOADS["clip_241f"]
    _say("case clip_241f (27,280 tokens x 20 heads)")
    inp = make_inputs(w)
    o, st = _run(inp)
    o_ref, s_ref = oracle_for(inp)
    _check(inp, o, st, o_ref, s_ref, TOL_BF16, "clip_241f")


@pytest.mark.parametrize("T, reverse, workload", [(27240, False, "clip_241f"), (27240, True, "clip_241f"),
                                                   (27223, False, "clip_241f_fp8")])
def test_ragged_last_chunk_full_width(T, reverse, workload):
    """340 full chunks and a last chunk of 40 (23) rows, 20 heads: in the last
    chunk range the state pass's copy waves issue row loads and row touches
    with lanes past the sequence's end.  Every head against the oracle, and
    three calls bitwise equal."""
    from oracle import bidirectional as BD
    inp = make_inputs(WORKLOADS[workload], seq_len=T)
    _say(f"case ragged last chunk: {workload} T={T} reverse={reverse}")
    q, k, v, g, beta, s0 = to_device(inp)
    runs = []
    for _ in range(3):
        o, st = gdn.gdn_fwd(q, k, v, g, beta, s0, reverse=reverse)
        torch.cuda.synchronize()
        runs.append((o, st))
    for o, st in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(st, runs[0][1])
    args = (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.state0)
    o_ref, s_ref = BD.reverse_scan(*args) if reverse else oracle_for(inp)
    _check(inp, runs[0][0].cpu().numpy(), runs[0][1].cpu().numpy(), o_ref, s_ref, TOL_BF16,
           f"ragged last chunk {workload} T={T} reverse={reverse}")


@pytest.mark.parametrize("reverse", [False, True])
def test_more_state_workgroups_than_cus(reverse):
    """B = 4 x 24 heads: 96 (b, h) units, so 384 state-pass workgroups, more
    than the 256 CUs, which then do not all run at once (no workgroup waits on
    another, so the order they run in does not matter).  A ragged 1,999-token
    sequence with an entry state; every unit against the oracle, and two calls
    bitwise equal."""
    from oracle import bidirectional as BD
    from hybrid_linear_attention_gdn_amd.inputs import Workload
    w = Workload("wide", 4, 24, 1, 10**9, "bf16", 31, state_std=0.02)
    inp = make_inputs(w, seq_len=1999, frame_tokens=880)
    _say(f"case 4 x 24 heads, T=1999, reverse={reverse}")
    q, k, v, g, beta, s0 = to_device(inp)
    o1, st1 = gdn.gdn_fwd(q, k, v, g, beta, s0, reverse=reverse)
    o2, st2 = gdn.gdn_fwd(q, k, v, g, beta, s0, reverse=reverse)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(st1, st2)
    args = (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.state0)
    o_ref, s_ref = BD.reverse_scan(*args) if reverse else oracle_for(inp)
    _check(inp, o1.cpu().numpy(), st1.cpu().numpy(), o_ref, s_ref, TOL_BF16, f"4 x 24 heads reverse={reverse}")


def test_streaming_rollout_equals_one_pass():
    w = WORKLOADS["stream_3f_x10"]
    _say("case stream_3f_x10: 10 chunk steps of 2,640 tokens")
    inp = make_inputs(w)
    q, k, v, g, beta, s0 = to_device(inp)
    Tc = w.tokens_per_call
    state = s0.clone()
    outs = []
    for c in range(w.calls):
        sl = slice(c * Tc, (c + 1) * Tc)
        o, state = gdn.gdn_chunk_step(q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous(),
                                      g[:, sl].contiguous(), beta[:, sl].contiguous(), state, state)
        outs.append(o)
    o_roll = torch.cat(outs, 1)
    o_one, s_one = gdn.gdn_fwd(q, k, v, g, beta, s0)
    torch.cuda.synchronize()
    assert torch.equal(o_roll, o_one), "rollout differs from one pass"
    assert torch.equal(state, s_one)
    o_ref, s_ref = oracle_for(inp)
    _check(inp, o_one.cpu().numpy(), s_one.cpu().numpy(), o_ref, s_ref, TOL_BF16, "stream_3f_x10")


def test_minute_cfg_all_units():
    """B = 2, 106,480 tokens: the GPU runs the full problem; the oracle checks
    every one of the 40 (b, h) units, element by element (about a minute of
    the host's cores)."""
    w = WORKLOADS["minute_cfg"]
    _say("case minute_cfg (2 x 106,480 tokens x 20 heads)")
    inp = make_inputs(w)
    o, st = _run(inp)
    assert np.isfinite(o).all()
    for b in range(2):
        o_ref, s_ref = oracle_for(inp, batches=[b])
        _check(inp, o[[b]], st[[b]], o_ref, s_ref, TOL_BF16, f"minute_cfg b={b}, all 20 heads")
        del o_ref, s_ref


def test_batch_copies_equal_single_batch():
    """B = 2 x 20 heads: twice the state-pass workgroups of B = 1, so a
    different split of the merged launches between state pass and intra-chunk
    work.  With batch 1 a copy of batch 0, both must equal the B = 1 result
    bit for bit (a ragged 5,063-token sequence with an initial state)."""
    w = WORKLOADS["clip_241f"]
    inp = make_inputs(w, seq_len=5063)
    inp.state0 = (0.02 * np.random.default_rng(7).standard_normal((1, 20, 112, 112))).astype(np.float32)
    q, k, v, g, beta, s0 = to_device(inp)
    _say("case batch copies: B=2 vs B=1, T=5063")
    o1, st1 = gdn.gdn_fwd(q, k, v, g, beta, s0)
    cat = lambda t: torch.cat([t, t], 0).contiguous()  # noqa: E731
    o2, st2 = gdn.gdn_fwd(cat(q), cat(k), cat(v), cat(g), cat(beta), cat(s0))
    torch.cuda.synchronize()
    assert torch.equal(o2[:1], o1) and torch.equal(o2[1:], o1)
    assert torch.equal(st2[:1], st1) and torch.equal(st2[1:], st1)
    o_ref, s_ref = oracle_for(inp, heads=[0, 19], batches=[0])
    _check(inp, o1.cpu().numpy()[:, :, [0, 19]], st1.cpu().numpy()[:, [0, 19]], o_ref, s_ref, TOL_BF16,
           "batch copies, heads 0 and 19")


def test_closed_forms_on_gpu():
    from hybrid_linear_attention_gdn_amd.inputs import Workload
    w = Workload("closed", 1, 2, 2, 100, "bf16", 77)
    inp = make_inputs(w)
    # beta = 0 (logit -inf), zero state: nothing is written, o = 0 exactly
    inp.beta[:] = -np.inf
    for fp32 in (False, True):
        o, st = _run(inp, fp32=fp32)
        assert not o.any() and not st.any()
    # alpha = 1, beta = 1, distinct standard-basis keys, every query = key 0: o_t = v_0 for all t
    T = 112
    w2 = Workload("basis", 1, 1, 1, T, "bf16", 78)
    inp2 = make_inputs(w2, seq_len=T)
    perm = np.random.default_rng(0).permutation(112)
    inp2.k[:] = 0
    inp2.k[0, np.arange(T), 0, perm[:T]] = 1.0
    inp2.q[:] = inp2.k[:, :1]
    inp2.g[:] = 0
    inp2.beta[:] = np.inf
    from hybrid_linear_attention_gdn_amd.inputs import round_bf16_bits
    inp2.q_bits, inp2.k_bits = round_bf16_bits(inp2.q), round_bf16_bits(inp2.k)
    for fp32 in (False, True):
        o, st = _run(inp2, fp32=fp32)
        np.testing.assert_allclose(o[0, :, 0], np.repeat(inp2.v[0, :1, 0], T, 0), rtol=0, atol=1e-5)
        np.testing.assert_allclose(st[0, 0] @ inp2.k[0, :, 0].T, inp2.v[0, :, 0].T, rtol=0, atol=1e-5)


def test_prep_scalars_match_definitions():
    """Standalone prep kernel outputs (fp32 path, read from the workspace) against their
    definitions in fp64; the MFMA path's per-chunk scalars are checked in test_gpu_kernels."""
    w = WORKLOADS["window_2f"]
    inp = make_inputs(w, seq_len=250)
    q, k, v, g, beta, _ = to_device(inp, fp32=True)
    p = gdn.problem(1, 250, 20, 112, 112, torch.float32, torch.float32)
    lay = gdn.workspace_layout(p)
    ws = torch.empty(lay.total, dtype=torch.uint8, device="cuda")
    gdn.gdn_fwd(q, k, v, g, beta, workspace=ws)
    torch.cuda.synchronize()
    f = lambda off: ws[off:off + 4 * 20 * 250].view(torch.float32).view(1, 20, 250).cpu().numpy()  # noqa: E731
    bt, rq, rk, gc = f(lay.beta), f(lay.rq), f(lay.rk), f(lay.gcum)
    tr = lambda a: np.transpose(a, (0, 2, 1)).astype(np.float64)  # noqa: E731  [B,T,H] -> [B,H,T]
    np.testing.assert_allclose(bt, 1 / (1 + np.exp(-tr(inp.beta))), rtol=2e-6)
    np.testing.assert_allclose(rq, 1 / np.linalg.norm(np.transpose(inp.q, (0, 2, 1, 3)), axis=-1), rtol=2e-6)
    np.testing.assert_allclose(rk, 1 / np.linalg.norm(np.transpose(inp.k, (0, 2, 1, 3)), axis=-1), rtol=2e-6)
    G = tr(inp.g).reshape(1, 20, 250)
    ref = np.concatenate([np.cumsum(G[..., c:c + 80], -1) for c in range(0, 250, 80)], -1)
    np.testing.assert_allclose(gc, ref, rtol=1e-6, atol=1e-6)


def test_determinism_aliasing_and_empty():
    w = WORKLOADS["window_2f"]
    inp = make_inputs(w, seq_len=400)
    inp.state0 = (0.02 * np.random.default_rng(1).standard_normal((1, 20, 112, 112))).astype(np.float32)
    q, k, v, g, beta, s0 = to_device(inp)
    o1, st1 = gdn.gdn_fwd(q, k, v, g, beta, s0)
    o2, st2 = gdn.gdn_fwd(q, k, v, g, beta, s0)
    s_inplace = s0.clone()
    o3, _ = gdn.gdn_fwd(q, k, v, g, beta, s_inplace, s_inplace)
    o4, none = gdn.gdn_fwd(q, k, v, g, beta, s0, None)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(st1, st2)
    assert torch.equal(o3, o1) and torch.equal(s_inplace, st1)
    assert torch.equal(o4, o1) and none is None
    # empty sequence: state passes through
    e = lambda t: t[:, :0].contiguous()  # noqa: E731
    oe, se = gdn.gdn_fwd(e(q), e(k), e(v), e(g), e(beta), s0)
    oz, sz = gdn.gdn_fwd(e(q), e(k), e(v), e(g), e(beta), None)
    torch.cuda.synchronize()
    assert oe.shape == (1, 0, 20, 112) and torch.equal(se, s0) and not sz.any()


def test_bf16_output_mode():
    """bf16 o: the path's own rounding of o (RNE) -- checked against the fp32-o result."""
    w = WORKLOADS["window_2f"]
    inp = make_inputs(w)
    o32, _ = _run(inp)
    o16, _ = _run(inp, o_dtype=torch.bfloat16)
    from hybrid_linear_attention_gdn_amd.inputs import round_bf16
    # rounding fp32 -> bf16 is one ulp at most away from the RNE of the fp32 result
    ulp = np.abs(round_bf16(o32) - o32).max()
    assert np.max(np.abs(o16 - round_bf16(o32))) <= 2 * ulp + 1e-30


def test_python_binding_rejects_bad_tensors():
    q = torch.zeros(1, 80, 2, 112, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(1, 80, 2, device="cuda")
    with pytest.raises(ValueError):
        gdn.gdn_fwd(q, q, q, g[:, :40], g)
    with pytest.raises(TypeError):
        gdn.gdn_fwd(q, q.float(), q, g, g)
    with pytest.raises(gdn.GdnError):
        gdn.gdn_chunk_step(q[:, :50].contiguous(), q[:, :50].contiguous(), q[:, :50].contiguous(),
                           g[:, :50].contiguous(), g[:, :50].contiguous(), torch.zeros(1, 2, 112, 112, device="cuda"))
