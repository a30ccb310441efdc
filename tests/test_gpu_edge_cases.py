"""Edge cases of the gated delta rule on both kernel families (bf16 inputs on
the MFMA kernels, the same values as fp32 on the vector-ALU kernels) and both
scan directions, against the fp64 oracle (oracle/recurrence.py,
oracle/bidirectional.py).

* decays of exactly zero (g = -inf) and of e^-200 in the middle of a chunk and
  on a chunk's first token: the kernels floor g at -80, which changes such a
  decay by at most e^-80 (the state before it is forgotten either way);
* rows of q or k that are exactly zero (normalised as x / max(||x||, eps):
  the row stays zero, a zero query reads exactly 0);
* dense per-token gates -softplus(N(0,1) + 2) at the full 241-frame shape,
  every head;
* retrieval of a stored value with standard-basis keys, alpha = beta = 1:
  exact, so asserted bit for bit;
* a NaN gate: the documented reading is that NaN propagates -- every output of
  the NaN's chunk from its token on and every later output is NaN (the
  chunked kernels may also turn the chunk's earlier rows NaN), the outputs of
  earlier chunks are untouched.
Bars: 1e-2 of rms(o_ref) on the MFMA kernels, 1e-4 on the fp32 kernels.
"""
import sys

import numpy as np
import pytest
import torch

from hybrid_linear_attention_gdn_amd import gdn
from hybrid_linear_attention_gdn_amd.inputs import (WORKLOADS, Workload, bf16_bits_to_f32, make_inputs,
                                                    round_bf16_bits)
from oracle import bidirectional as BD
from oracle.recurrence import gdn_recurrence
from tests.helpers import TOL_BF16, TOL_F32, rel_max_err, state_err, to_device

pytestmark = pytest.mark.gpu

FAMILIES = [False, True]  # fp32 inputs: False = MFMA kernels, True = vector-ALU kernels
DIRECTIONS = [False, True]  # reverse scan


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _refresh_bits(inp):
    inp.q_bits, inp.k_bits, inp.v_bits = (round_bf16_bits(a) for a in (inp.q, inp.k, inp.v))


def _run(inp, fp32, reverse, s_in=None):
    q, k, v, g, beta, s0 = to_device(inp, fp32=fp32)
    if s_in is not None:
        s0 = torch.from_numpy(s_in).cuda()
    o, st = gdn.gdn_fwd(q, k, v, g, beta, s0, reverse=reverse)
    torch.cuda.synchronize()
    return o.cpu().numpy(), st.cpu().numpy()


def _oracle(inp, reverse, heads=None, s_in=None):
    sel = lambda a: a if heads is None else a[:, :, heads]  # noqa: E731
    s0 = inp.state0 if s_in is None else s_in
    if s0 is not None and heads is not None:
        s0 = s0[:, heads]
    args = [sel(a) for a in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
    return BD.reverse_scan(*args, s0) if reverse else gdn_recurrence(*args, s0)


def _check(o, st, o_ref, s_ref, fp32, label):
    tol = TOL_F32 if fp32 else TOL_BF16
    eo, es = rel_max_err(o, o_ref), state_err(st, s_ref)
    _say(f"[{label}] o {eo:.3e} state {es:.3e} (bar {tol:g})")
    assert np.isfinite(o).all() and np.isfinite(st).all()
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("fp32", FAMILIES)
@pytest.mark.parametrize("reverse", DIRECTIONS)
def test_infinite_and_deep_decays_mid_chunk(fp32, reverse):
    w = Workload("deep_gates", 1, 4, 1, 10**9, "bf16", 501, state_std=0.05)
    inp = make_inputs(w, seq_len=410, frame_tokens=41)  # frame-wise gates every 41 tokens
    inp.g[0, 37, 0] = -np.inf     # mid-chunk, head 0
    inp.g[0, 80, 1] = -np.inf     # a chunk's first token, head 1
    inp.g[0, 203, 2] = -200.0     # mid-chunk, head 2
    inp.g[0, 160, 3] = -200.0     # a chunk's first token, head 3
    inp.g[0, 409, 0] = -np.inf    # the last token (the reverse scan never uses its gate)
    _say(f"case -inf / -200 gates, fp32 inputs={fp32}, reverse={reverse}")
    o, st = _run(inp, fp32, reverse)
    o_ref, s_ref = _oracle(inp, reverse)
    _check(o, st, o_ref, s_ref, fp32, "deep gates")


@pytest.mark.parametrize("fp32", FAMILIES)
@pytest.mark.parametrize("reverse", DIRECTIONS)
def test_zero_query_and_key_rows(fp32, reverse):
    w = Workload("zero_rows", 1, 3, 1, 10**9, "bf16", 502, state_std=0.05)
    inp = make_inputs(w, seq_len=250, frame_tokens=83)
    zq = [0, 37, 79, 80, 249]
    zk = [1, 38, 80, 81, 159, 248]
    inp.q[0, zq] = 0.0
    inp.k[0, zk] = 0.0
    _refresh_bits(inp)
    _say(f"case zero q rows {zq}, zero k rows {zk}, fp32 inputs={fp32}, reverse={reverse}")
    o, st = _run(inp, fp32, reverse)
    assert not o[0, zq].any(), "a zero query must read exactly 0"
    o_ref, s_ref = _oracle(inp, reverse)
    _check(o, st, o_ref, s_ref, fp32, "zero rows")


@pytest.mark.parametrize("fp32", FAMILIES)
@pytest.mark.parametrize("reverse", DIRECTIONS)
def test_dense_per_token_gates_full_shape(fp32, reverse):
    """Per-token gates -softplus(N(0,1) + 2) (frame length 1) on the 241-frame
    shape, 27,280 tokens x 20 heads; the oracle checks every head."""
    w = WORKLOADS["clip_241f"]
    inp = make_inputs(w, frame_tokens=1)
    assert (inp.g < 0).all()
    _say(f"case dense gates 27,280 x 20, fp32 inputs={fp32}, reverse={reverse}")
    o, st = _run(inp, fp32, reverse)
    assert np.isfinite(o).all()
    o_ref, s_ref = _oracle(inp, reverse)
    _check(o, st, o_ref, s_ref, fp32, "dense gates, all 20 heads")


@pytest.mark.parametrize("fp32", FAMILIES)
@pytest.mark.parametrize("reverse", DIRECTIONS)
def test_standard_basis_retrieval_is_exact(fp32, reverse):
    """alpha = beta = 1, the 112 standard-basis keys in a random order over
    T = 112 tokens (a full chunk and a ragged one); every query is the key of
    token 0 (forward) or of token T - 1 (reverse), so every o_t is that token's
    value and the exit state is sum_t v_t k_t^T, all exactly.  Values are kept
    at magnitude >= 2^-8 so that they are exact in every operand format the
    kernels use."""
    T, d = 112, 112
    w = Workload("basis", 1, 1, 1, T, "bf16", 503)
    inp = make_inputs(w, seq_len=T)
    perm = np.random.default_rng(5).permutation(d)
    inp.k[:] = 0.0
    inp.k[0, np.arange(T), 0, perm] = 1.0
    src = T - 1 if reverse else 0
    inp.q[:] = inp.k[:, src:src + 1]
    v = inp.v
    inp.v = (np.sign(v) * np.maximum(np.abs(v), 2.0 ** -8)).astype(np.float32)
    _refresh_bits(inp)
    inp.v = v_exact = bf16_bits_to_f32(inp.v_bits)
    inp.g[:] = 0.0
    inp.beta[:] = np.inf
    _say(f"case standard-basis retrieval, fp32 inputs={fp32}, reverse={reverse}")
    o, st = _run(inp, fp32, reverse)
    np.testing.assert_array_equal(o[0, :, 0], np.repeat(v_exact[0, src:src + 1, 0], T, 0))
    S = np.zeros((d, d), np.float32)  # S[i, j] = v_t[i] where k_t = e_j
    S[:, perm] = v_exact[0, :, 0].T
    np.testing.assert_array_equal(st[0, 0], S)


@pytest.mark.parametrize("fp32", FAMILIES)
def test_nan_gate_propagates(fp32):
    """The NaN reading: a NaN log-decay at token 117 (chunk 1) of head 1 turns
    o of head 1 NaN from token 117 on and its exit state NaN; chunk 0 of that
    head and every other head equal the clean run bit for bit.  In the reverse
    scan the same gate is the decay between tokens 116 and 117: o of head 1 is
    NaN up to token 116, and from token 197 (past the NaN's chunk) it equals
    the clean run."""
    w = Workload("nan_gate", 1, 3, 1, 10**9, "bf16", 504, state_std=0.05)
    inp = make_inputs(w, seq_len=250, frame_tokens=50)
    o0, s0 = _run(inp, fp32, False)
    r0, _ = _run(inp, fp32, True)
    inp.g[0, 117, 1] = np.nan
    _say(f"case NaN gate, fp32 inputs={fp32}")
    o, st = _run(inp, fp32, False)
    assert np.isnan(o[0, 117:, 1]).all() and np.isnan(st[0, 1]).all()
    np.testing.assert_array_equal(o[0, :80, 1], o0[0, :80, 1])
    for h in (0, 2):
        np.testing.assert_array_equal(o[:, :, h], o0[:, :, h])
        np.testing.assert_array_equal(st[:, h], s0[:, h])
    r, _ = _run(inp, fp32, True)
    assert np.isnan(r[0, :117, 1]).all()
    np.testing.assert_array_equal(r[0, 197:, 1], r0[0, 197:, 1])
    np.testing.assert_array_equal(r[:, :, [0, 2]], r0[:, :, [0, 2]])
