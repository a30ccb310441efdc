"""Pins of the fp64 attention-block oracle (oracle/attention.py) to values fixed
by the mathematics and by the stream geometry the pages give (SGLang cookbook
page "SANA-WM", section "Configuration reference": 3 frames per block, 2
cached blocks, 1 sink frame), not by the oracle itself."""
import math

import numpy as np
import pytest

from oracle import attention as A


@pytest.mark.parametrize("block,expected", [
    # 3 frames per block, 2 cached blocks, 1 sink frame: enumerated by hand
    (0, [0, 1, 2]),
    (1, [0, 1, 2, 3, 4, 5]),
    (2, [0, 1, 2, 3, 4, 5, 6, 7, 8]),
    (3, [0, 3, 4, 5, 6, 7, 8, 9, 10, 11]),
    (4, [0, 6, 7, 8, 9, 10, 11, 12, 13, 14]),
    (9, [0, 21, 22, 23, 24, 25, 26, 27, 28, 29]),
])
def test_context_frames_page_geometry(block, expected):
    assert A.context_frames(block, 3, 2, 1) == expected


def test_context_frames_other_geometries():
    assert A.context_frames(4, 3, 2, 0) == list(range(6, 15))            # no sink
    assert A.context_frames(3, 3, 2, 4) == list(range(0, 12))            # sink overlaps the window
    assert A.context_frames(5, 1, 0, 1) == [0, 5]                        # no cache: sink + current
    assert A.context_frames(0, 3, 2, 5) == [0, 1, 2]                     # sink frames not yet generated
    with pytest.raises(ValueError):
        A.context_frames(-1, 3, 2, 1)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    q, k, v = rng.normal(size=(5, 8)), rng.normal(size=(1, 8)), rng.normal(size=(1, 6))
    np.testing.assert_array_equal(A.attention(q, k, v), np.repeat(v, 5, axis=0))


def test_zero_query_averages_values():
    rng = np.random.default_rng(2)
    k, v = rng.normal(size=(7, 8)), rng.normal(size=(7, 3))
    np.testing.assert_allclose(A.attention(np.zeros((2, 8)), k, v), np.repeat(v.mean(0, keepdims=True), 2, 0),
                               rtol=0, atol=1e-15)


def test_scale_is_one_over_sqrt_d():
    # logits differ by ln 2 only under the 1/sqrt(d) scale: weights 2/3 and 1/3
    d = 9
    q = np.zeros((1, d))
    q[0, 0] = math.log(2.0) * math.sqrt(d)
    k = np.zeros((2, d))
    k[0, 0] = 1.0
    v = np.array([[3.0, 0.0], [0.0, 3.0]])
    np.testing.assert_allclose(A.attention(q, k, v), [[2.0, 1.0]], rtol=0, atol=1e-14)


def test_common_key_shift_and_key_order_do_not_matter():
    rng = np.random.default_rng(3)
    q, k, v = rng.normal(size=(4, 16)), rng.normal(size=(11, 16)), rng.normal(size=(11, 5))
    o = A.attention(q, k, v)
    u = rng.normal(size=(1, 16))
    # q . (k_j + u) = q . k_j + q . u: the same shift for every key of a query row
    np.testing.assert_allclose(A.attention(q, k + u, v), o, rtol=0, atol=1e-12)
    perm = rng.permutation(11)
    np.testing.assert_allclose(A.attention(q, k[perm], v[perm]), o, rtol=0, atol=1e-14)


def test_dominant_key_limit():
    # a logit gap of 800 leaves the other weights below the fp64 underflow: exact
    d = 4
    q = np.zeros((1, d))
    q[0, 1] = 800.0 * math.sqrt(d)
    k = np.array([[0.0, 1.0, 0.0, 0.0], [0.0, 0.0, 1.0, 0.0], [1.0, 0.0, 0.0, 0.0]])
    v = np.array([[1.5, -2.0], [7.0, 7.0], [9.0, 9.0]])
    np.testing.assert_array_equal(A.attention(q, k, v), [[1.5, -2.0]])


def test_stream_block_attends_each_context_frame_once():
    # zero queries weigh every context key equally; values one-hot by frame
    # index give the share of each frame: 1/10 for the 10 frames of block 4
    ft, fpb, C, S = 2, 3, 2, 1
    nblocks, H = 5, 2
    frames = nblocks * fpb
    T = frames * ft
    kh = np.random.default_rng(4).normal(size=(1, T, H, 8))
    vh = np.zeros((1, T, H, frames))
    for f in range(frames):
        vh[0, f * ft:(f + 1) * ft, :, f] = 1.0
    q = np.zeros((1, fpb * ft, H, 8))
    o = A.stream_block(q, kh, vh, 4, ft, fpb, C, S)
    want = np.zeros(frames)
    want[[0, 6, 7, 8, 9, 10, 11, 12, 13, 14]] = 0.1
    np.testing.assert_allclose(o[0, 3, 1], want, rtol=0, atol=1e-15)
