"""GPU parity of the reverse scan (GDN_FLAG_REVERSE) and of the bidirectional
layer (gdn_bidir_fwd) against the fp64 oracle (oracle/bidirectional.py), on
both kernel families.  Bars as for the forward scan: 1e-2 of rms(o_ref) with
bf16 or fp8 inputs, 1e-4 on the fp32 path, the exit state against its rms."""
import sys

import numpy as np
import pytest
import torch

from hybrid_linear_attention_gdn_amd import gdn
from hybrid_linear_attention_gdn_amd.inputs import WORKLOADS, Workload, make_inputs, round_bf16
from oracle import bidirectional as BD
from tests.helpers import TOL_BF16, TOL_F32, rel_max_err, state_err, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check(got, ref, tol, label, st=None, s_ref=None):
    eo = rel_max_err(got, ref)
    es = state_err(st, s_ref) if st is not None else 0.0
    _say(f"[{label}] max|o-o_ref|/rms = {eo:.3e}   state: {es:.3e}   (bar {tol:g})")
    assert np.isfinite(got).all()
    assert eo <= tol and es <= tol, (eo, es)


def _sel(inp, heads=None, t_end=None):
    arrs = [inp.q, inp.k, inp.v, inp.g, inp.beta]
    if t_end is not None:
        arrs = [a[:, :t_end] for a in arrs]
    if heads is not None:
        arrs = [a[:, :, heads] for a in arrs]
    return arrs


@pytest.mark.parametrize("fp32", [False, True])
def test_reverse_scan_window_2f(fp32):
    w = WORKLOADS["window_2f"]
    inp = make_inputs(w)
    s_in = (0.02 * np.random.default_rng(21).standard_normal((1, 20, 112, 112))).astype(np.float32)
    _say("case reverse scan window_2f fp32 inputs=", fp32)
    q, k, v, g, beta, _ = to_device(inp, fp32=fp32)
    o, st = gdn.gdn_fwd(q, k, v, g, beta, torch.from_numpy(s_in).cuda(), reverse=True)
    torch.cuda.synchronize()
    o_ref, s_ref = BD.reverse_scan(*_sel(inp), s_in)
    _check(o.cpu().numpy(), o_ref, TOL_BF16, "reverse window_2f", st.cpu().numpy(), s_ref)


@pytest.mark.parametrize("T,B,H", [(1, 1, 2), (79, 1, 3), (81, 2, 2), (250, 1, 4), (401, 2, 3)])
def test_reverse_scan_ragged(T, B, H):
    w = Workload("ragged_rev", B, H, 1, 10**9, "bf16", 60 + T, state_std=0.05)
    inp = make_inputs(w, seq_len=T, frame_tokens=97)
    _say("case reverse ragged", T, B, H)
    o_ref, s_ref = BD.reverse_scan(*_sel(inp), inp.state0)
    for fp32 in (False, True):
        q, k, v, g, beta, s0 = to_device(inp, fp32=fp32)
        o, st = gdn.gdn_fwd(q, k, v, g, beta, s0, reverse=True)
        torch.cuda.synchronize()
        _check(o.cpu().numpy(), o_ref, TOL_BF16, f"reverse T={T} fp32 inputs={fp32}", st.cpu().numpy(), s_ref)


def test_reverse_scan_fp32_portable():
    w = WORKLOADS["tiny_fp32"]
    inp = make_inputs(w, seq_len=250)
    q, k, v, g, beta, s0 = to_device(inp)
    _say("case reverse tiny_fp32 (T=250)")
    o, st = gdn.gdn_fwd(q, k, v, g, beta, s0, reverse=True)
    torch.cuda.synchronize()
    o_ref, s_ref = BD.reverse_scan(*_sel(inp), inp.state0)
    _check(o.cpu().numpy(), o_ref, TOL_F32, "reverse fp32", st.cpu().numpy(), s_ref)


def test_reverse_batch_copies_equal_single_batch():
    """B = 2 x 20 heads (another split of the merged launches than B = 1): both
    batches must equal the B = 1 result bit for bit."""
    w = WORKLOADS["clip_241f"]
    inp = make_inputs(w, seq_len=5063)
    s_in = (0.02 * np.random.default_rng(22).standard_normal((1, 20, 112, 112))).astype(np.float32)
    q, k, v, g, beta, _ = to_device(inp)
    s0 = torch.from_numpy(s_in).cuda()
    _say("case reverse, batch copies: B=2 vs B=1, T=5063")
    o1, st1 = gdn.gdn_fwd(q, k, v, g, beta, s0, reverse=True)
    cat = lambda t: torch.cat([t, t], 0).contiguous()  # noqa: E731
    o2, st2 = gdn.gdn_fwd(cat(q), cat(k), cat(v), cat(g), cat(beta), cat(s0), reverse=True)
    torch.cuda.synchronize()
    assert torch.equal(o2[:1], o1) and torch.equal(o2[1:], o1)
    assert torch.equal(st2[:1], st1) and torch.equal(st2[1:], st1)
    o_ref, s_ref = BD.reverse_scan(*_sel(inp, heads=[0, 19]), s_in[:, [0, 19]])
    _check(o1.cpu().numpy()[:, :, [0, 19]], o_ref, TOL_BF16, "reverse batch copies, heads 0 and 19",
           st1.cpu().numpy()[:, [0, 19]], s_ref)


@pytest.mark.parametrize("fp32", [False, True])
def test_bidir_window_2f(fp32):
    w = WORKLOADS["window_2f"]
    inp = make_inputs(w)
    _say("case bidirectional window_2f fp32 inputs=", fp32)
    q, k, v, g, beta, _ = to_device(inp, fp32=fp32)
    o = gdn.gdn_bidir_fwd(q, k, v, g, beta)
    o16 = gdn.gdn_bidir_fwd(q, k, v, g, beta, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    _check(o, BD.bidirectional(*_sel(inp)), TOL_BF16, "bidirectional window_2f")
    # bf16 o: the one rounding of the same fp32 sum
    np.testing.assert_array_equal(o16.float().cpu().numpy(), round_bf16(o))


@pytest.mark.parametrize("fp32", [False, True])
def test_bidir_equals_forward_plus_reverse_bitwise(fp32):
    # o is the one fp32 sum of the two scans' outputs (formed as the reverse
    # scan stores, or by the combine kernel); each scan alone is gdn_fwd with
    # and without GDN_FLAG_REVERSE
    w = Workload("bidir_sum", 1, 4, 3, 210, "bf16", 91)  # T = 630: seven full chunks and a ragged one
    inp = make_inputs(w)
    q, k, v, g, beta, _ = to_device(inp, fp32=fp32)
    _say("case bidirectional = forward + reverse, fp32 inputs=", fp32)
    o = gdn.gdn_bidir_fwd(q, k, v, g, beta)
    of, _ = gdn.gdn_fwd(q, k, v, g, beta, state_out=None)
    orv, _ = gdn.gdn_fwd(q, k, v, g, beta, state_out=None, reverse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, of + orv)


def test_bidir_batch_copies_equal_single_batch():
    """The bidirectional layer at B = 2 x 20 heads with batch 1 a copy of batch
    0: both batches equal the B = 1 layer bit for bit (ragged T = 5,063)."""
    w = WORKLOADS["clip_241f"]
    inp = make_inputs(w, seq_len=5063)
    q, k, v, g, beta, _ = to_device(inp)
    _say("case bidirectional, batch copies: B=2 vs B=1, T=5063")
    o1 = gdn.gdn_bidir_fwd(q, k, v, g, beta)
    cat = lambda t: torch.cat([t, t], 0).contiguous()  # noqa: E731
    o2 = gdn.gdn_bidir_fwd(cat(q), cat(k), cat(v), cat(g), cat(beta))
    torch.cuda.synchronize()
    assert torch.equal(o2[:1], o1) and torch.equal(o2[1:], o1)
    o_ref = BD.bidirectional(*_sel(inp, heads=[0, 19]))
    _check(o1.cpu().numpy()[:, :, [0, 19]], o_ref, TOL_BF16, "bidirectional batch copies, heads 0 and 19")


@pytest.mark.parametrize("T", [1, 81, 250])
def test_bidir_ragged_and_fp32(T):
    w = Workload("ragged_bidir", 2, 3, 1, 10**9, "bf16", 70 + T)
    inp = make_inputs(w, seq_len=T, frame_tokens=97)
    q, k, v, g, beta, _ = to_device(inp)
    _say("case bidirectional ragged", T)
    o = gdn.gdn_bidir_fwd(q, k, v, g, beta)
    torch.cuda.synchronize()
    _check(o.cpu().numpy(), BD.bidirectional(*_sel(inp)), TOL_BF16, f"bidirectional T={T}")
    w32 = WORKLOADS["tiny_fp32"]
    inp32 = make_inputs(w32, seq_len=T)
    q, k, v, g, beta, _ = to_device(inp32)
    o = gdn.gdn_bidir_fwd(q, k, v, g, beta)
    torch.cuda.synchronize()
    _check(o.cpu().numpy(), BD.bidirectional(*_sel(inp32)), TOL_F32, f"bidirectional fp32 T={T}")


def test_bidir_fp8_equals_bf16_on_the_same_values():
    w = WORKLOADS["window_2f_fp8"]
    inp = make_inputs(w)
    q, k, v, g, beta, _ = to_device(inp)
    _say("case bidirectional fp8 == bf16")
    o8 = gdn.gdn_bidir_fwd(q, k, v, g, beta)
    b16 = lambda t: t.float().to(torch.bfloat16)  # noqa: E731  exact for E4M3FN values
    o16 = gdn.gdn_bidir_fwd(b16(q), b16(k), b16(v), g, beta)
    torch.cuda.synchronize()
    assert torch.equal(o8, o16)
    _check(o8.cpu().numpy(), BD.bidirectional(*_sel(inp)), TOL_BF16, "bidirectional fp8")


def test_bidir_clip_241f_all_heads():
    """The 27,280-token layer, both scans; the oracle checks all 20 heads."""
    w = WORKLOADS["clip_241f"]
    inp = make_inputs(w)
    q, k, v, g, beta, _ = to_device(inp)
    _say("case bidirectional clip_241f, all heads")
    o = gdn.gdn_bidir_fwd(q, k, v, g, beta)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    assert np.isfinite(o).all()
    _check(o, BD.bidirectional(*_sel(inp)), TOL_BF16, "bidirectional clip_241f, all 20 heads")


def test_bidir_deterministic_and_empty():
    w = WORKLOADS["window_2f"]
    inp = make_inputs(w, seq_len=400)
    q, k, v, g, beta, _ = to_device(inp)
    a = gdn.gdn_bidir_fwd(q, k, v, g, beta)
    b = gdn.gdn_bidir_fwd(q, k, v, g, beta)
    e = lambda t: t[:, :0].contiguous()  # noqa: E731
    z = gdn.gdn_bidir_fwd(e(q), e(k), e(v), e(g), e(beta))
    torch.cuda.synchronize()
    assert torch.equal(a, b) and z.shape == (1, 0, 20, 112)
    with pytest.raises(gdn.GdnError):
        gdn.gdn_chunk_step(q[:, :320].contiguous(), k[:, :320].contiguous(), v[:, :320].contiguous(),
                           g[:, :320].contiguous(), beta[:, :320].contiguous(),
                           torch.zeros(1, 20, 112, 112, device="cuda"), reverse=True)
