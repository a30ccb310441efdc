"""gdn_fwd_no_alloc (the entry point on the library's fixed per-device
workspace) against gdn_fwd on the same inputs, through the C ABI.  Its chunk
ranges are shorter (they must fit 64 MiB), and the state carried between
ranges is exact fp32, so the outputs must equal gdn_fwd's bit for bit.  Two
calls and more in a row, each smaller than the one before, reuse the array."""
import sys

import pytest
import torch

from hybrid_linear_attention_gdn_amd import gdn
from hybrid_linear_attention_gdn_amd.inputs import WORKLOADS, Workload, make_inputs
from tests.helpers import TOL_BF16, oracle_for, rel_max_err, state_err, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _both(inp, fp32=False, o_dtype=torch.float32, reverse=False):
    q, k, v, g, beta, s0 = to_device(inp, fp32=fp32)
    B, T, H, d = q.shape
    o_ref, st_ref = gdn.gdn_fwd(q, k, v, g, beta, s0, o_dtype=o_dtype, reverse=reverse)
    o = torch.full((B, T, H, d), float("nan"), dtype=o_dtype, device="cuda")
    st = torch.full((B, H, d, d), float("nan"), dtype=torch.float32, device="cuda")
    gdn.gdn_fwd_no_alloc(q, k, v, g, beta, s0, st, o, reverse=reverse)
    torch.cuda.synchronize()
    return o, st, o_ref, st_ref


def test_no_alloc_equals_gdn_fwd_on_shrinking_calls():
    # 1: the 241-frame clip (341 chunks: 15 launches in ranges of at most 26 chunks)
    w = WORKLOADS["clip_241f"]
    inp = make_inputs(w)
    _say("case no-alloc 1: clip_241f, B=1 T=27280 H=20")
    o, st, o_ref, st_ref = _both(inp)
    assert torch.equal(o, o_ref) and torch.equal(st, st_ref)
    oc, sc = oracle_for(inp, heads=[0, 19])
    e = rel_max_err(o.cpu().numpy()[:, :, [0, 19]], oc)
    _say(f"   max|o-o_ref|/rms heads 0, 19 = {e:.3e}")
    assert e <= TOL_BF16
    # 2: smaller, ragged, with an initial state, B = 2
    w2 = Workload("na2", 2, 6, 1, 10**9, "bf16", 301, state_std=0.05)
    inp2 = make_inputs(w2, seq_len=1013, frame_tokens=97)
    _say("case no-alloc 2: B=2 T=1013 H=6, initial state")
    o, st, o_ref, st_ref = _both(inp2)
    assert torch.equal(o, o_ref) and torch.equal(st, st_ref)
    o_or, s_or = oracle_for(inp2)
    assert rel_max_err(o.cpu().numpy(), o_or) <= TOL_BF16 and state_err(st.cpu().numpy(), s_or) <= TOL_BF16
    # 3: smaller still: the reverse scan, bf16 o
    inp3 = make_inputs(w2, seq_len=250, frame_tokens=97)
    _say("case no-alloc 3: B=2 T=250 H=6 reverse, bf16 o")
    o, st, o_ref, st_ref = _both(inp3, o_dtype=torch.bfloat16, reverse=True)
    assert torch.equal(o, o_ref) and torch.equal(st, st_ref)
    # 4: the fp32 kernels on a problem whose whole workspace fits
    inp4 = make_inputs(WORKLOADS["tiny_fp32"])
    _say("case no-alloc 4: tiny_fp32 (vector-ALU kernels)")
    o, st, o_ref, st_ref = _both(inp4, fp32=True)
    assert torch.equal(o, o_ref) and torch.equal(st, st_ref)


def test_no_alloc_rejects_what_does_not_fit():
    # B * H = 400 units need more than 64 MiB even with one-chunk ranges
    q = torch.zeros(1, 80, 400, 112, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(1, 80, 400, device="cuda")
    o = torch.empty(1, 80, 400, 112, device="cuda")
    with pytest.raises(gdn.GdnError, match="workspace"):
        gdn.gdn_fwd_no_alloc(q, q, q, g, g, None, None, o)
    # the fp32 kernels' workspace grows with T: 20 heads x 27,280 tokens does not fit
    q32 = torch.zeros(1, 27280, 20, 112, device="cuda")
    g32 = torch.zeros(1, 27280, 20, device="cuda")
    with pytest.raises(gdn.GdnError, match="workspace"):
        gdn.gdn_fwd_no_alloc(q32, q32, q32, g32, g32, None, None, q32.clone())
