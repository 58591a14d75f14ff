"""Pins of the oracle's planner and conv stem: counts against the pages'
printed shapes, brute-force convolution, torch fp64 conv2d, locality, PE."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_shapes.json")))


def test_after_cnn_len_is_ceil_of_eighth():
    for m in range(1, 2000):
        assert O.after_cnn_len(m) == -(-m // 8)
    assert O.after_cnn_len(GOLD["chunk_tokens"]["frames"]) == GOLD["chunk_tokens"]["tokens"]


def test_counts_against_printed_shapes():
    assert O.after_cnn_len(100) * 8 == GOLD["window_tokens"]["value"]
    # 9 full chunks -> 117 tokens
    assert O.clip_num_tokens(9 * 100 * 160) == GOLD["win_9_chunks"]["tokens"]
    # 20 minutes -> 15600 tokens, which fits the ~122 pages of 128 tokens
    t20 = O.clip_num_tokens(GOLD["twenty_minutes"]["samples"])
    assert t20 == 15600
    pages = GOLD["twenty_minutes"]["pages_of_128_tokens"]
    assert (pages - 1) * 128 < t20 <= pages * 128
    assert O.clip_num_tokens(480000) == 390
    assert O.clip_num_tokens(32000) == 26
    assert O.clip_num_tokens(0) == 0
    # tail chunks: 26 frames -> 4 tokens, 1 frame -> 1 token
    assert O.clip_num_tokens(126 * 160) == 13 + 4
    assert O.clip_num_tokens(101 * 160) == 13 + 1


def test_windows_cover_tokens():
    for n in (0, 1, 103, 104, 105, 15600, 5986):
        wb = O.window_bounds(n)
        assert sum(e - s for s, e in wb) == n
        assert all(0 < e - s <= 104 for s, e in wb)


def _conv_brute(x, w, b):
    cin, h, wd = x.shape
    cout = w.shape[0]
    ho, wo = (h + 1) // 2, (wd + 1) // 2
    z = np.zeros((cout, ho, wo))
    for co in range(cout):
        for i in range(ho):
            for j in range(wo):
                s = b[co]
                for ci in range(cin):
                    for a in range(3):
                        for bb in range(3):
                            r, c = 2 * i + a - 1, 2 * j + bb - 1
                            if 0 <= r < h and 0 <= c < wd:
                                s += w[co, ci, a, bb] * x[ci, r, c]
                z[co, i, j] = s
    return z


@pytest.mark.parametrize("shape", [(1, 8, 10), (3, 8, 10), (2, 7, 5)])
def test_conv_brute_force(shape):
    rng = np.random.default_rng(4)
    x = rng.standard_normal(shape)
    w = rng.standard_normal((2, shape[0], 3, 3))
    b = rng.standard_normal(2)
    assert np.allclose(O.conv2d_k3s2p1(x, w, b), _conv_brute(x, w, b), atol=1e-12)


def test_conv_matches_torch_fp64():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 128, 100))
    w = rng.standard_normal((5, 6, 3, 3))
    b = rng.standard_normal(5)
    ref = torch.nn.functional.conv2d(torch.from_numpy(x)[None], torch.from_numpy(w),
                                     torch.from_numpy(b), stride=2, padding=1)[0].numpy()
    z = O.conv2d_k3s2p1(x, w, b)
    assert z.shape == (5, 64, 50)
    assert np.allclose(z, ref, atol=1e-11)


def test_gelu_is_erf_gelu():
    z = np.linspace(-6, 6, 1001)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="none").numpy()
    assert np.allclose(O.gelu(z), ref, atol=1e-15)
    assert O.gelu(np.array([0.0]))[0] == 0.0
    tanh = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    assert np.abs(O.gelu(z) - tanh).max() > 1e-4       # not the tanh flavour


def _tiny_stem_weights(C=4, d=8, seed=6):
    rng = np.random.default_rng(seed)
    return {"conv1_w": rng.standard_normal((C, 1, 3, 3)) * 0.3, "conv1_b": rng.standard_normal(C) * 0.1,
            "conv2_w": rng.standard_normal((C, C, 3, 3)) * 0.3, "conv2_b": rng.standard_normal(C) * 0.1,
            "conv3_w": rng.standard_normal((C, C, 3, 3)) * 0.3, "conv3_b": rng.standard_normal(C) * 0.1,
            "conv_out_w": rng.standard_normal((d, C * 16)) * 0.1}


def test_stem_matches_torch_pipeline():
    W = _tiny_stem_weights()
    rng = np.random.default_rng(7)
    mel = rng.standard_normal((128, 100))
    t = torch.from_numpy(mel)[None, None]
    for l in (1, 2, 3):
        t = torch.nn.functional.gelu(torch.nn.functional.conv2d(
            t, torch.from_numpy(W[f"conv{l}_w"]), torch.from_numpy(W[f"conv{l}_b"]), stride=2, padding=1))
    b, c, f, tt = t.shape
    v = t.permute(0, 3, 1, 2).reshape(b, tt, c * f)        # channel outer, frequency inner
    ref = (v @ torch.from_numpy(W["conv_out_w"]).T)[0].numpy()
    got = O.stem_chunk(mel, W, 100)
    assert got.shape == (13, 8)
    assert np.allclose(got, ref, atol=1e-11)


def test_stem_flatten_order_channel_outer():
    # a conv_out that reads only feature c*16+f = 1*16+3 picks channel 1, frequency 3
    W = _tiny_stem_weights()
    W["conv_out_w"] = np.zeros_like(W["conv_out_w"])
    W["conv_out_w"][0, 1 * 16 + 3] = 1.0
    mel = np.random.default_rng(8).standard_normal((128, 100))
    z = mel[None]
    for l in (1, 2, 3):
        z = O.gelu(O.conv2d_k3s2p1(z, W[f"conv{l}_w"], W[f"conv{l}_b"]))
    got = O.stem_chunk(mel, W, 100)
    assert np.allclose(got[:, 0], z[1, 3, :], atol=1e-14)


def test_tail_readings_agree_on_full_chunks_and_differ_on_tail():
    W = _tiny_stem_weights()
    mel = np.random.default_rng(9).standard_normal((128, 100))
    assert np.array_equal(O.stem_chunk(mel, W, 100, "A"), O.stem_chunk(mel, W, 100, "B"))
    a = O.stem_chunk(mel[:, :37], W, 37, "A")
    b = O.stem_chunk(mel[:, :37], W, 37, "B")
    assert a.shape == b.shape == (5, 8)
    assert np.allclose(a[:3], b[:3], atol=1e-12)      # far from the padded edge
    assert not np.allclose(a[-1], b[-1])


def test_pe_closed_forms():
    pe = O.sinusoid_pe(13, 256)
    assert np.all(pe[0, :128] == 0.0) and np.all(pe[0, 128:] == 1.0)
    t = np.arange(13)
    assert np.allclose(pe[:, 0], np.sin(t), atol=1e-15)
    assert np.allclose(pe[:, 128], np.cos(t), atol=1e-15)
    # the slowest frequency is 1/10000
    assert np.allclose(pe[:, 127], np.sin(t * 1e-4), atol=1e-15)
    assert np.allclose(pe[:, :128] ** 2 + pe[:, 128:] ** 2, 1.0, atol=1e-14)
