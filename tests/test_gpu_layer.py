"""GPU parity of the layer around the scan (include/sanawm_gdn.h, "The layer
around the scan"): the two projection kernels against fp64 products of the
same bf16 values, and the whole layer against the fp64 layer oracle
(oracle/layer.py).

Bars.  A projection accumulates K = H*112 exact bf16 x bf16 products in fp32,
so |c - c_ref| <= K 2^-24 sum_k |a_k w_k| (the worst-case bound of recursive
fp32 summation); bf16 outputs add their own rounding, 2^-8 |c_ref|.  The gate
g = -softplus(a) moves by at most |delta a| plus fp32 rounding of the softplus.
The layer: max |y - y_ref| <= 1e-2 rms(y_ref), the scan's bar, against the
oracle that stores q, k, v and o in bf16 as the bf16 model does (plus 2^-8
|y_ref| per element for bf16 y).  The error against the unrounded fp64 layer is
reported beside it, with the distance of the bf16-storage oracle from that
layer: the storage roundings alone move y by about 2e-2 of rms."""
import sys

import numpy as np
import pytest
import torch

from hybrid_linear_attention_gdn_amd import gdn, layer
from hybrid_linear_attention_gdn_amd.inputs import make_layer_inputs
from oracle import layer as LY
from tests.helpers import state_err

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _up(bits):
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def _fp32_bound(a, w):
    """K 2^-24 sum_k |a_k w_k| for every output element of a w^T."""
    K = a.shape[-1]
    return K * 2.0 ** -24 * (np.abs(a.astype(np.float64)) @ np.abs(w.astype(np.float64)).T)


@pytest.mark.parametrize("B,T,H", [(1, 1, 20), (1, 255, 20), (2, 257, 4), (1, 1000, 20), (1, 300, 3)])
def test_in_proj(B, T, H):
    ft = 97
    li = make_layer_inputs(B, T, H, ft, 400 + T + H)
    _say("case in_proj", B, T, H)
    q, k, v, beta, g = layer.in_proj(_up(li.x_bits), _up(li.w_in_bits), ft)
    torch.cuda.synchronize()
    rq, rk, rv, rbeta, rg = LY.in_proj(li.x, li.w_in, H, ft)
    bound = _fp32_bound(li.x, li.w_in)  # [B, T, N]
    HD = H * 112
    for name, got, ref, cols in (("q", q, rq, slice(0, HD)), ("k", k, rk, slice(HD, 2 * HD)),
                                 ("v", v, rv, slice(2 * HD, 3 * HD))):
        got = got.float().cpu().numpy().reshape(B, T, HD)
        ref = ref.reshape(B, T, HD)
        err = np.abs(got - ref) - (bound[..., cols] + 2.0 ** -8 * np.abs(ref))
        assert err.max() <= 0, (name, err.max())
    b_cols = slice(3 * HD, 3 * HD + H)
    assert (np.abs(beta.cpu().numpy() - rbeta) <= bound[..., b_cols]).all()
    gg = g.cpu().numpy()
    first = (np.arange(T) % ft == 0)
    assert not gg[:, ~first].any()
    slack = bound[..., 3 * HD + H:] + 2.0 ** -20 * (1 + np.abs(rg))
    assert (np.abs(gg - rg) <= slack)[:, first].all()


@pytest.mark.parametrize("B,T,H,y_dtype", [(1, 1, 20, torch.float32), (1, 513, 20, torch.float32),
                                           (2, 300, 4, torch.bfloat16), (1, 1000, 20, torch.bfloat16)])
def test_out_proj(B, T, H, y_dtype):
    li = make_layer_inputs(B, T, H, 1, 500 + T + H)
    _say("case out_proj", B, T, H, y_dtype)
    y = layer.out_proj(_up(li.x_bits), _up(li.w_out_bits), y_dtype=y_dtype)
    torch.cuda.synchronize()
    ref = li.x.astype(np.float64) @ li.w_out.astype(np.float64).T
    slack = _fp32_bound(li.x, li.w_out) + (2.0 ** -8 * np.abs(ref) if y_dtype == torch.bfloat16 else 0.0)
    err = np.abs(y.float().cpu().numpy() - ref) - slack
    assert err.max() <= 0, err.max()


@pytest.mark.parametrize("bidir", [False, True])
def test_layer_matches_oracle(bidir):
    B, T, H, ft = 1, 1760, 20, 880
    li = make_layer_inputs(B, T, H, ft, 600 + bidir)
    s_in = None if bidir else (0.02 * np.random.default_rng(6).standard_normal((B, H, 112, 112))).astype(np.float32)
    _say("case layer window_2f bidirectional=", bidir)
    st_in = None if bidir else torch.from_numpy(s_in).cuda()
    st_out = None if bidir else torch.empty_like(st_in)
    y, st = layer.layer_fwd(_up(li.x_bits), _up(li.w_in_bits), _up(li.w_out_bits), ft, st_in, st_out,
                            bidirectional=bidir)
    torch.cuda.synchronize()
    y_ref, s_ref = LY.layer(li.x, li.w_in, li.w_out, H, ft, s_in, bidirectional_scan=bidir)
    y = y.cpu().numpy()
    err = np.abs(y - y_ref).max() / np.sqrt(np.mean(y_ref ** 2))
    _say(f"layer bidir={bidir}: max |y - y_ref| / rms = {err:.3e} (bar {TOL})")
    assert err <= TOL
    # reported beside the bar: the layer with no bf16 storage at all, and how far
    # the bf16-storage oracle itself is from it (the kernel cannot be closer to
    # the unrounded layer than about that)
    y_x, _ = LY.layer(li.x, li.w_in, li.w_out, H, ft, s_in, bidirectional_scan=bidir, bf16_intermediates=False)
    rms_x = np.sqrt(np.mean(y_x ** 2))
    err_x = np.abs(y - y_x).max() / rms_x
    storage = np.abs(y_ref - y_x).max() / rms_x
    _say(f"  against the unrounded fp64 layer: {err_x:.3e}; bf16-storage oracle against it: {storage:.3e}")
    assert err_x <= storage + TOL
    if not bidir:
        es = state_err(st.cpu().numpy(), s_ref)
        _say(f"exit state: {es:.3e}")
        assert es <= TOL


def test_layer_ragged_bf16_output():
    B, T, H, ft = 2, 173, 4, 50
    li = make_layer_inputs(B, T, H, ft, 700)
    y, _ = layer.layer_fwd(_up(li.x_bits), _up(li.w_in_bits), _up(li.w_out_bits), ft, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y_ref, _ = LY.layer(li.x, li.w_in, li.w_out, H, ft)
    # bf16 y: the bar plus the rounding of y itself, 2^-8 |y_ref| per element
    rms = np.sqrt(np.mean(y_ref ** 2))
    score = (np.abs(y.float().cpu().numpy() - y_ref) / (TOL * rms + 2.0 ** -8 * np.abs(y_ref))).max()
    _say(f"layer ragged bf16 y: max |y - y_ref| / (1e-2 rms + 2^-8 |y_ref|) = {score:.3f}")
    assert score <= 1.0


def test_layer_page_shape_sampled_rows():
    """The 27,280-token layer equals its three calls composed (in_proj, the
    scan with bf16 o, out_proj) bit for bit; the projections are checked on
    sampled rows against fp64 products of the same bf16 values (the GPU's own
    o for the out-projection)."""
    B, T, H, ft = 1, 27280, 20, 880
    li = make_layer_inputs(B, T, H, ft, 800)
    x, w_in, w_out = _up(li.x_bits), _up(li.w_in_bits), _up(li.w_out_bits)
    _say("case layer clip_241f (27,280 tokens)")
    y, _ = layer.layer_fwd(x, w_in, w_out, ft)
    q, k, v, beta, g = layer.in_proj(x, w_in, ft)
    o, _ = gdn.gdn_fwd(q, k, v, g, beta, None, None, o_dtype=torch.bfloat16)
    y2 = layer.out_proj(o, w_out)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    HD = H * 112
    rows = np.random.default_rng(9).choice(T, 64, replace=False)
    rq, _, _, rbeta, _ = LY.in_proj(li.x[:, rows], li.w_in, H, 1)
    b = _fp32_bound(li.x[:, rows], li.w_in)
    rq = rq.reshape(1, 64, HD)
    qs = q.float().cpu().numpy()[:, rows].reshape(1, 64, HD)
    assert (np.abs(qs - rq) <= b[..., :HD] + 2.0 ** -8 * np.abs(rq)).all()
    assert (np.abs(beta.cpu().numpy()[:, rows] - rbeta) <= b[..., 3 * HD:3 * HD + H]).all()
    gg = g.cpu().numpy()
    assert not gg[:, np.arange(T) % ft != 0].any() and (gg[:, ::ft] < 0).all()
    o_rows = o.float().cpu().numpy()[:, rows].reshape(1, 64, HD)
    y_ref = o_rows.astype(np.float64) @ li.w_out.astype(np.float64).T
    assert (np.abs(y.cpu().numpy()[:, rows] - y_ref) <= _fp32_bound(o_rows, li.w_out)).all()
    assert np.isfinite(y.cpu().numpy()).all()
