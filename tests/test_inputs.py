"""Host-side checks of the seeded input generator (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from hybrid_linear_attention_gdn_amd import inputs as I


def test_page_shapes(golden_dir):
    gd = json.load(open(os.path.join(golden_dir, "page_shapes.json")))
    assert I.tokens_per_frame(gd["frame"]["height"], gd["frame"]["width"]) == gd["frame"]["latent_tokens"]
    for px, lat in gd["pixel_to_latent_frames"]:
        assert I.latent_frames(px) == lat
    assert I.HEADS == gd["heads"] and I.HEAD_DIM == gd["head_dim"] and I.HEADS * I.HEAD_DIM == gd["hidden"]
    w = I.WORKLOADS["stream_3f_x10"]
    assert w.tokens_per_call == gd["streaming_call_tokens"] == gd["streaming_block_latent_frames"] * 880
    assert I.WORKLOADS["clip_241f"].seq_len == 27280
    assert I.WORKLOADS["minute_cfg"].seq_len == 106480 and I.WORKLOADS["minute_cfg"].batch == 2
    with pytest.raises(ValueError):
        I.latent_frames(240)


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10.0 ** r.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9 * 3,
                                  np.inf, -np.inf, 3.4e38, 1e-40], np.float32)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(I.round_bf16_bits(x), ref)
    assert np.array_equal(I.round_bf16(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_determinism_and_recipe():
    w = I.WORKLOADS["window_2f"]
    a = I.make_inputs(w, seq_len=1760)
    b = I.make_inputs(w, seq_len=1760)
    for n in ("q", "k", "v", "g", "beta"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
    assert a.q.shape == (1, 1760, 20, 112) and a.g.shape == (1, 1760, 20)
    # frame-wise gate: non-zero only on the first token of each 880-token frame, always < 0
    nz = np.nonzero(a.g[0, :, 0])[0]
    assert list(nz) == [0, 880]
    assert (a.g[0, [0, 880]] < 0).all()
    # q, k, v hold bf16-exact values
    assert np.array_equal(I.round_bf16(a.q), a.q)
    assert np.array_equal(I.bf16_bits_to_f32(a.q_bits), a.q)
    c = I.make_inputs(w, seed=5, seq_len=1760)
    assert not np.array_equal(c.q, a.q)
    s = I.make_inputs(I.WORKLOADS["stream_3f_x10"], seq_len=880, frame_tokens=880)
    assert s.state0.shape == (1, 20, 112, 112) and 0.015 < s.state0.std() < 0.025
    t = I.make_inputs(I.WORKLOADS["tiny_fp32"])
    assert t.q_bits is None and t.q.dtype == np.float32 and t.q.shape == (1, 320, 4, 112)


# ---- E4M3FN (OCP 8-bit floating point): values fixed by the format's definition
from hybrid_linear_attention_gdn_amd.inputs import e4m3_codes_to_f32, round_e4m3_codes  # noqa: E402


def test_e4m3_landmark_codes():
    dec = e4m3_codes_to_f32(np.arange(256, dtype=np.uint8))
    assert dec[0x00] == 0.0 and np.signbit(dec[0x80])
    assert dec[0x01] == 2.0 ** -9          # smallest subnormal
    assert dec[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert dec[0x08] == 2.0 ** -6          # smallest normal
    assert dec[0x38] == 1.0 and dec[0xC0] == -2.0 and dec[0x39] == 1.125
    assert dec[0x7E] == 448.0 and dec[0xFE] == -448.0
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    finite = dec[np.isfinite(dec)]
    assert finite.size == 254


def test_e4m3_rounding():
    codes = round_e4m3_codes(np.array([1.0, 1.0625, 1.1875, 1.09, 500.0, -1e-4, 2.0 ** -10, 3 * 2.0 ** -10,
                                       -448.0, np.nan], np.float32))
    # 1.0625 is halfway between 1 (even) and 1.125: even; 1.1875 halfway between 1.125 and 1.25 (even)
    assert list(codes[:4]) == [0x38, 0x38, 0x3A, 0x39]
    assert codes[4] == 0x7E                    # saturates at 448
    assert codes[5] == 0x80                    # rounds to -0
    assert codes[6] == 0x00 and codes[7] == 0x02  # subnormal ties to even: 0.5 -> 0, 1.5 -> 2 (x 2^-9)
    assert codes[8] == 0xFE and codes[9] == 0x7F


def test_e4m3_round_trip_every_finite_code():
    c = np.arange(256, dtype=np.uint8)
    c = c[(c & 0x7F) != 0x7F]
    np.testing.assert_array_equal(round_e4m3_codes(e4m3_codes_to_f32(c)), c)
