"""Pins of the oracle's encoder: LayerNorm invariants, windowed attention
identities, identity layers, and whole-forward special cases with a closed
form, plus an independent torch-fp64 composition on a small encoder."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth


def test_layer_norm_invariants_and_torch():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((7, 96)) * 3 + 1
    g = np.ones(96)
    b = np.zeros(96)
    y = O.layer_norm(x, g, b)
    var = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-13)
    assert np.allclose(y.var(axis=1), 1.0 / (1.0 + O.LN_EPS / var), rtol=1e-12)
    g = rng.standard_normal(96)
    b = rng.standard_normal(96)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    assert np.allclose(O.layer_norm(x, g, b), ref, atol=1e-12)


def _qkv(t, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((t, d)) for _ in range(3)]


def test_attention_matches_torch_sdpa_block_mask():
    q, k, v = _qkv(30, 128, 11)
    segs = [(0, 13), (13, 26), (26, 30)]
    o = np.empty_like(q)
    for s, e in segs:
        o[s:e] = O.mha(q[s:e], k[s:e], v[s:e], 2)
    mask = torch.zeros(30, 30, dtype=torch.bool)
    for s, e in segs:
        mask[s:e, s:e] = True
    tq = torch.from_numpy(q).view(30, 2, 64).transpose(0, 1)
    tk = torch.from_numpy(k).view(30, 2, 64).transpose(0, 1)
    tv = torch.from_numpy(v).view(30, 2, 64).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    ref = ref.transpose(0, 1).reshape(30, 128).numpy()
    assert np.allclose(o, ref, atol=1e-12)


def test_attention_identities():
    q, k, v = _qkv(20, 64, 12)
    # constant V -> output is that constant
    vc = np.tile(np.arange(64.0), (20, 1))
    assert np.allclose(O.mha(q, k, vc, 1), vc, atol=1e-12)
    # rows of the attention matrix sum to 1
    a = O.softmax(q @ k.T / 8.0)
    assert np.allclose(a.sum(axis=1), 1.0, atol=1e-14)
    # permutation equivariance inside a window
    p = np.random.default_rng(13).permutation(20)
    assert np.allclose(O.mha(q[p], k[p], v[p], 1), O.mha(q, k, v, 1)[p], atol=1e-12)
    # scale 1/sqrt(head_dim): with two identical keys and q.k known, weights follow
    q1 = np.zeros((1, 64)); q1[0, 0] = 8.0
    k1 = np.zeros((2, 64)); k1[0, 0] = 1.0
    v1 = np.array([[1.0] + [0.0] * 63, [0.0] * 64])
    out = O.mha(q1, k1, v1, 1)
    assert out[0, 0] == pytest.approx(math.e / (math.e + 1.0), abs=1e-14)


def _small_weights(d=64, heads=2, ffn=128, C=8, out=48, layers=2, seed=14, std=0.1):
    dims = synth.Dims(conv_channels=C, d_model=d, n_layers=layers, n_heads=heads, head_dim=d // heads,
                      ffn_dim=ffn, output_dim=out, dtype="f32")
    return dims, O.as_f64(synth.make_weights(dims, seed, std))


def test_windowed_equals_separate_and_window_isolation():
    dims, W = _small_weights()
    L = O.layer_weights(W, 0)
    rng = np.random.default_rng(15)
    x = rng.standard_normal((250, 64))
    segs = O.window_bounds(250)
    y = O.encoder_layer(x, L, segs, 2)
    for s, e in segs:
        assert np.allclose(y[s:e], O.encoder_layer(x[s:e], L, [(0, e - s)], 2), atol=1e-12)
    x2 = x.copy()
    x2[120] += 1.0                       # perturb a token of window 1
    y2 = O.encoder_layer(x2, L, segs, 2)
    assert np.array_equal(y2[:104], y[:104]) and np.array_equal(y2[208:], y[208:])
    assert not np.allclose(y2[104:208], y[104:208])


def test_zero_layer_is_identity():
    dims, W = _small_weights()
    L = {k: np.zeros_like(v) for k, v in O.layer_weights(W, 0).items()}
    x = np.random.default_rng(16).standard_normal((40, 64))
    assert np.array_equal(O.encoder_layer(x, L, [(0, 40)], 2), x)


def test_whole_forward_identity_special_case():
    # zero stem and zero layers: every token is its chunk-local PE row; with
    # unit LayerNorm and identity projections the output is gelu(LN(PE[j])).
    d = 64
    dims, W = _small_weights(d=d, out=d)
    for k in W:
        if k.startswith("conv") or k.startswith("layers."):
            W[k] = np.zeros_like(W[k])
    W["post_ln_w"], W["post_ln_b"] = np.ones(d), np.zeros(d)
    W["proj1_w"], W["proj1_b"] = np.eye(d), np.zeros(d)
    W["proj2_w"], W["proj2_b"] = np.eye(d), np.zeros(d)
    n = 160 * 1234 + 77                   # 1234 frames: 12 full chunks + 34-frame tail
    x = np.random.default_rng(17).standard_normal(n)
    out = O.encode([x], W, 2, 2)
    pe = O.sinusoid_pe(13, d)
    expect_rows = [pe[j] for _ in range(12) for j in range(13)] + [pe[j] for j in range(5)]
    expect = O.gelu(O.layer_norm(np.array(expect_rows), np.ones(d), np.zeros(d)))
    assert out.shape == (12 * 13 + 5, d)
    assert np.allclose(out, expect, atol=1e-12)


def _torch_forward(x, W, dims):
    """Independent composition from torch fp64 library ops (conv2d, layer_norm,
    scaled_dot_product_attention with a block mask, gelu) and numpy.fft."""
    tt = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    xp = np.pad(x.astype(np.float64), 200, mode="reflect")
    n_fr = 1 + (xp.shape[0] - 400) // 160
    w = np.hanning(401)[:400]             # periodic Hann = first N of the N+1 symmetric window
    fr = np.stack([xp[160 * j:160 * j + 400] for j in range(n_fr)])
    p = np.abs(np.fft.rfft(fr * w, axis=1)) ** 2
    lg = np.log10(np.maximum(p @ O.mel_filterbank().T, 1e-10))[:-1].T
    mel = (np.maximum(lg, lg.max() - 8) + 4) / 4
    F = mel.shape[1]
    toks = []
    for c0 in range(0, F, 100):
        m = min(100, F - c0)
        img = np.zeros((128, 100)); img[:, :m] = mel[:, c0:c0 + m]
        t = tt(img)[None, None]
        for l in (1, 2, 3):
            t = torch.nn.functional.gelu(torch.nn.functional.conv2d(
                t, tt(W[f"conv{l}_w"]), tt(W[f"conv{l}_b"]), stride=2, padding=1))
        v = t.permute(0, 3, 1, 2).reshape(t.shape[3], -1) @ tt(W["conv_out_w"]).T
        pos = torch.arange(13, dtype=torch.float64)[:, None]
        half = dims.d_model // 2
        inv = torch.exp(-math.log(10000.0) / (half - 1) * torch.arange(half, dtype=torch.float64))
        pe = torch.cat([torch.sin(pos * inv), torch.cos(pos * inv)], dim=1)
        toks.append((v + pe)[: -(-m // 8)])
    h = torch.cat(toks)
    T = h.shape[0]
    mask = torch.zeros(T, T, dtype=torch.bool)
    for s in range(0, T, 104):
        mask[s:s + 104, s:s + 104] = True
    D, H = dims.d_model, dims.n_heads
    for l in range(dims.n_layers):
        g = lambda n: tt(W[f"layers.{l}.{n}"])
        a = torch.nn.functional.layer_norm(h, (D,), g("ln1_w"), g("ln1_b"), eps=1e-5)
        q = torch.nn.functional.linear(a, g("q_w"), g("q_b")).view(T, H, -1).transpose(0, 1)
        k = torch.nn.functional.linear(a, g("k_w"), g("k_b")).view(T, H, -1).transpose(0, 1)
        v = torch.nn.functional.linear(a, g("v_w"), g("v_b")).view(T, H, -1).transpose(0, 1)
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
        h = h + torch.nn.functional.linear(o.transpose(0, 1).reshape(T, D), g("o_w"), g("o_b"))
        a = torch.nn.functional.layer_norm(h, (D,), g("ln2_w"), g("ln2_b"), eps=1e-5)
        u = torch.nn.functional.gelu(torch.nn.functional.linear(a, g("fc1_w"), g("fc1_b")))
        h = h + torch.nn.functional.linear(u, g("fc2_w"), g("fc2_b"))
    a = torch.nn.functional.layer_norm(h, (D,), tt(W["post_ln_w"]), tt(W["post_ln_b"]), eps=1e-5)
    u = torch.nn.functional.gelu(torch.nn.functional.linear(a, tt(W["proj1_w"]), tt(W["proj1_b"])))
    return torch.nn.functional.linear(u, tt(W["proj2_w"]), tt(W["proj2_b"])).numpy()


def test_whole_forward_matches_independent_torch_composition():
    dims, W = _small_weights(d=128, heads=2, ffn=256, C=8, out=96, layers=2, std=0.05)
    x = synth.speech_like_clip(16000 * 17 + 4321, [99, 0])   # 17.27 s: 17 chunks + tail, 2 windows + ragged
    got = O.encode([x], W, dims.n_layers, dims.n_heads)
    ref = _torch_forward(x, W, dims)
    assert got.shape == ref.shape == (O.clip_num_tokens(x.shape[0]), 96)
    assert np.allclose(got, ref, atol=1e-9, rtol=1e-9)


def test_packed_batch_is_clipwise():
    dims, W = _small_weights()
    xs = [synth.speech_like_clip(n, [98, i]) for i, n in enumerate((3000, 17000, 0, 40000))]
    packed = O.encode(xs, W, 2, 2)
    parts = [O.encode([x], W, 2, 2) for x in xs]
    assert np.array_equal(packed, np.concatenate(parts))
    assert packed.shape[0] == sum(O.clip_num_tokens(len(x)) for x in xs)


def test_full_input_attention_reading():
    # window_chunks = 0: one attention segment over the whole clip; equal to
    # the windowed forward whenever the clip fits one window, different (and
    # window-coupled) beyond it; clips over 30 s are refused.
    dims, W = _small_weights()
    short = synth.speech_like_clip(16000 * 5, [97, 0])          # 65 tokens < 104
    a = O.encode_clip(short, W, 2, 2, window_chunks=0)
    b = O.encode_clip(short, W, 2, 2, window_chunks=8)
    assert np.allclose(a[0], b[0], atol=1e-12)
    long = synth.speech_like_clip(16000 * 12, [97, 1])          # 156 tokens: 2 windows
    full = O.encode_clip(long, W, 2, 2, window_chunks=0)[0]
    win = O.encode_clip(long, W, 2, 2, window_chunks=8)
    assert full.shape[0] == 156 and not np.allclose(full[:104], win[0])
    x2 = long.copy(); x2[16000 * 11:] *= 0.5                    # touch only the last window's audio
    full2 = O.encode_clip(x2, W, 2, 2, window_chunks=0)[0]
    assert not np.allclose(full2[:52], full[:52])                # early rows see it under full attention
    with pytest.raises(O.InvalidInput):
        O.encode_clip(synth.speech_like_clip(30 * 16000 + 1, [97, 2]), W, 2, 2, window_chunks=0)
