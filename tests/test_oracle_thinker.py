"""Pins of the Thinker-prefill oracle ([qwenasr] "Qwen3 Thinker decoder",
"Prompt assembly and audio splice"): RMSNorm invariants, NEOX RoPE against an
independent complex-number rotation plus its relative-position property,
causal GQA attention against torch SDPA, SwiGLU against torch, the splice
rows, causality, identity layers, packed = separate prompts, and the whole
prefill against an independent torch fp64 composition."""
import numpy as np
import pytest
import torch

import oracle.thinker as TH
import synth.thinker as ST


def test_rms_norm_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)) * 3
    y = TH.rms_norm(x, np.ones(64), eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-14)
    assert np.allclose(TH.rms_norm(7.0 * x, np.ones(64), eps=0.0), y, atol=1e-14)   # scale invariant
    g = rng.standard_normal(64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(TH.rms_norm(x, g), ref, atol=1e-13)


def test_rope_neox_matches_complex_rotation_and_relative_property():
    rng = np.random.default_rng(2)
    T, H, d = 9, 3, 128
    x = rng.standard_normal((T, H, d))
    pos = np.arange(T) * 37
    y = TH.rope_neox(x, pos)
    # independent form: pair (i, i + 64) as the complex number x_i + j x_{i+64}
    h = d // 2
    z = x[..., :h] + 1j * x[..., h:]
    theta = 1e6 ** (-np.arange(h) / h)
    zr = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    assert np.allclose(y, np.concatenate([zr.real, zr.imag], axis=-1), atol=1e-12)
    assert np.allclose(TH.rope_neox(x, np.zeros(T)), x)                     # position 0 is identity
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))
    # <R(q, m), R(k, n)> depends only on m - n
    q, k = rng.standard_normal((1, 1, d)), rng.standard_normal((1, 1, d))
    a = (TH.rope_neox(q, [11]) * TH.rope_neox(k, [4])).sum()
    b = (TH.rope_neox(q, [1007]) * TH.rope_neox(k, [1000])).sum()
    assert a == pytest.approx(b, abs=1e-9)


def test_causal_gqa_matches_torch_sdpa():
    rng = np.random.default_rng(3)
    T, hq, hkv, d = 13, 4, 2, 128
    q, k, v = rng.standard_normal((T, hq, d)), rng.standard_normal((T, hkv, d)), rng.standard_normal((T, hkv, d))
    out = TH.causal_gqa(q, k, v)
    tq = torch.from_numpy(q).transpose(0, 1)
    tk = torch.from_numpy(k).transpose(0, 1).repeat_interleave(hq // hkv, dim=0)
    tv = torch.from_numpy(v).transpose(0, 1).repeat_interleave(hq // hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True).transpose(0, 1).numpy()
    assert np.allclose(out, ref, atol=1e-12)
    assert np.allclose(out[0], v[0][np.arange(hq) // 2])                   # token 0 sees only itself


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    assert np.allclose(TH.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), atol=1e-14)


def _small(seed=4, layers=2, std=0.05):
    d = ST.ThinkerDims(hidden=256, n_layers=layers, n_q_heads=2, n_kv_heads=1, ffn_dim=384, vocab=500,
                       dtype="f32")
    W = {k: v.astype(np.float64) for k, v in ST.make_weights(d, seed, std).items()}
    return d, W


def test_splice_rows_and_identity_layer():
    d, W = _small()
    ids, off = ST.make_prompt(7, d.vocab, [5, 0])
    audio = ST.make_audio_states(7, d.hidden, [5, 1]).astype(np.float64)
    x = TH.splice(ids, audio, off, W["embed"])
    assert np.array_equal(x[off:off + 7], audio)
    keep = np.r_[0:off, off + 7:ids.shape[0]]
    assert np.array_equal(x[keep], W["embed"][ids[keep]])
    L = {k: np.zeros_like(v) for k, v in TH.layer_weights(W, 0).items()}
    assert np.array_equal(TH.thinker_layer(x, L, 2, 1), x)


def test_causality_and_packed_batch():
    d, W = _small()
    ids, off = ST.make_prompt(5, d.vocab, [6, 0])
    audio = ST.make_audio_states(5, d.hidden, [6, 1]).astype(np.float64)
    h, lg = TH.prefill_prompt(ids, audio, off, W, 2, 2, 1)
    audio2 = audio.copy()
    audio2[-1] += 1.0                                    # change the last audio row
    h2, _ = TH.prefill_prompt(ids, audio2, off, W, 2, 2, 1)
    t = off + 4
    assert np.array_equal(h2[:t], h[:t]) and not np.allclose(h2[t:], h[t:])
    assert np.allclose(lg, W["embed"] @ h[-1])
    ids_b, off_b = ST.make_prompt(3, d.vocab, [6, 2])
    audio_b = ST.make_audio_states(3, d.hidden, [6, 3]).astype(np.float64)
    H, G = TH.prefill([(ids, audio, off), (ids_b, audio_b, off_b)], W, 2, 2, 1)
    hb, gb = TH.prefill_prompt(ids_b, audio_b, off_b, W, 2, 2, 1)
    assert np.array_equal(H, np.concatenate([h, hb])) and np.array_equal(G, np.stack([lg, gb]))


def _torch_prefill(ids, audio, off, W, d):
    """Independent composition from torch fp64 library ops."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    x = t(W["embed"])[torch.from_numpy(ids.astype(np.int64))].clone()
    x[off:off + audio.shape[0]] = t(audio)
    T = x.shape[0]
    hd = 128
    half = hd // 2
    inv = 1e6 ** (-torch.arange(half, dtype=torch.float64) / half)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None, :]
    cos, sin = torch.cat([ang.cos(), ang.cos()], 1), torch.cat([ang.sin(), ang.sin()], 1)

    def rot(u):                                           # rotate-half form, [H, T, hd]
        return u * cos + torch.cat([-u[..., half:], u[..., :half]], -1) * sin

    for l in range(d.n_layers):
        g = lambda n: t(W[f"layers.{l}.{n}"])
        a = torch.nn.functional.rms_norm(x, (d.hidden,), g("attn_norm"), eps=1e-6)
        q = torch.nn.functional.linear(a, g("q_w")).view(T, d.n_q_heads, hd)
        k = torch.nn.functional.linear(a, g("k_w")).view(T, d.n_kv_heads, hd)
        v = torch.nn.functional.linear(a, g("v_w")).view(T, d.n_kv_heads, hd)
        q = torch.nn.functional.rms_norm(q, (hd,), g("q_norm"), eps=1e-6).transpose(0, 1)
        k = torch.nn.functional.rms_norm(k, (hd,), g("k_norm"), eps=1e-6).transpose(0, 1)
        q, k = rot(q), rot(k)
        rep = d.n_q_heads // d.n_kv_heads
        o = torch.nn.functional.scaled_dot_product_attention(q, k.repeat_interleave(rep, 0),
                                                             v.transpose(0, 1).repeat_interleave(rep, 0),
                                                             is_causal=True)
        x = x + torch.nn.functional.linear(o.transpose(0, 1).reshape(T, -1), g("o_w"))
        a = torch.nn.functional.rms_norm(x, (d.hidden,), g("ffn_norm"), eps=1e-6)
        x = x + torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(a, g("gate_w")))
                                           * torch.nn.functional.linear(a, g("up_w")), g("down_w"))
    h = torch.nn.functional.rms_norm(x, (d.hidden,), t(W["out_norm"]), eps=1e-6)
    return h.numpy(), (h[-1] @ t(W["embed"]).T).numpy()


def test_prefill_matches_independent_torch_composition():
    d, W = _small(seed=7, layers=3)
    ids, off = ST.make_prompt(23, d.vocab, [8, 0])
    audio = ST.make_audio_states(23, d.hidden, [8, 1]).astype(np.float64)
    h, lg = TH.prefill_prompt(ids, audio, off, W, d.n_layers, d.n_q_heads, d.n_kv_heads)
    rh, rl = _torch_prefill(ids, audio, off, W, d)
    assert np.allclose(h, rh, atol=1e-10) and np.allclose(lg, rl, atol=1e-10)
