"""fp64 oracle of the audio splice and the Qwen3 Thinker prefill (test
infrastructure only).

Follows [qwenasr] "Qwen3 Thinker decoder" (per layer: RMSNorm -> q/k/v
projections -> per-head RMSNorm on q and k -> 1D NEOX RoPE -> attention over
the positions so far, GQA -> output projection, residual; RMSNorm -> SwiGLU
(silu(gate) * up) -> down projection, residual; final RMSNorm -> output
projection tied to the token embedding; no bias anywhere), "GGUF layout"
(16 query heads, 8 KV heads, head_dim 128, RoPE base 1e6) and "Prompt assembly
and audio splice" (embed the id sequence, then overwrite the S placeholder
rows with the encoder states).  [qwenasr] "Glossary" (NEOX RoPE: rotate-half
layout; the ASR timeline gives all three mrope axes the same id, so the rope is
plain 1D).

Readings (the pages leave these open):
* T1  rms_norm_eps is named but not valued; 1e-6.
* T2  prefill starts from an empty cache: positions 0 .. T-1 of each prompt,
      causal attention over [0, t] for token t.
* T3  the prefill returns the final-normed hidden states of every prompt token
      and the logits of each prompt's last token (what the first decode step
      samples from).
* T4  a packed batch of prompts never mixes: each prompt attends only to itself.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np

RMS_EPS = 1e-6          # reading T1
ROPE_BASE = 1e6         # [qwenasr] "GGUF layout": rope.freq_base 1e6
HEAD_DIM = 128          # [qwenasr] "GGUF layout": key_length / value_length 128


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis (RMSNorm, no bias)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope_neox(x: np.ndarray, pos: np.ndarray, base: float = ROPE_BASE) -> np.ndarray:
    """Rotate-half RoPE over the last axis (size 2h): the pair (x[i], x[i + h])
    is rotated by pos * base^(-i / h), i < h.  x: [T, heads, 2h]; pos: [T]."""
    h = x.shape[-1] // 2
    inv = base ** (-np.arange(h, dtype=np.float64) / h)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]      # [T, h]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def causal_gqa(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """q [T, Hq, d], k/v [T, Hkv, d]; query head h reads KV head h // (Hq / Hkv);
    token t attends to tokens 0..t; scale 1 / sqrt(d)."""
    T, hq, d = q.shape
    group = hq // k.shape[1]
    out = np.empty_like(q)
    mask = np.tril(np.ones((T, T), dtype=bool))
    for h in range(hq):
        kh, vh = k[:, h // group], v[:, h // group]
        s = q[:, h] @ kh.T / np.sqrt(d)
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h] = p @ vh
    return out


def layer_weights(W: Dict[str, np.ndarray], l: int) -> Dict[str, np.ndarray]:
    p = f"layers.{l}."
    return {k[len(p):]: v for k, v in W.items() if k.startswith(p)}


def thinker_layer(x: np.ndarray, L: Dict[str, np.ndarray], n_q: int, n_kv: int) -> np.ndarray:
    """One decoder layer over one prompt x [T, hidden] (positions 0..T-1)."""
    T = x.shape[0]
    d = HEAD_DIM
    a = rms_norm(x, L["attn_norm"])
    q = (a @ L["q_w"].T).reshape(T, n_q, d)
    k = (a @ L["k_w"].T).reshape(T, n_kv, d)
    v = (a @ L["v_w"].T).reshape(T, n_kv, d)
    q = rms_norm(q, L["q_norm"])                 # per head, over head_dim
    k = rms_norm(k, L["k_norm"])
    pos = np.arange(T)
    q = rope_neox(q, pos)
    k = rope_neox(k, pos)
    o = causal_gqa(q, k, v).reshape(T, n_q * d)
    x = x + o @ L["o_w"].T
    a = rms_norm(x, L["ffn_norm"])
    hdn = silu(a @ L["gate_w"].T) * (a @ L["up_w"].T)
    return x + hdn @ L["down_w"].T


def splice(ids: np.ndarray, audio: np.ndarray, audio_offset: int, embed: np.ndarray) -> np.ndarray:
    """Embed the id sequence, then overwrite rows audio_offset .. + S with the
    encoder states ([qwenasr] "Prompt assembly and audio splice")."""
    x = np.asarray(embed, dtype=np.float64)[np.asarray(ids)]
    S = audio.shape[0]
    if S:
        x[audio_offset:audio_offset + S] = audio
    return x


def prefill_prompt(ids: np.ndarray, audio: np.ndarray, audio_offset: int, W: Dict[str, np.ndarray],
                   n_layers: int, n_q: int, n_kv: int) -> Tuple[np.ndarray, np.ndarray]:
    """(hidden [T, hidden] after the final RMSNorm, logits [vocab] of the last
    token) for one prompt (readings T2, T3)."""
    x = splice(ids, audio, audio_offset, W["embed"])
    for l in range(n_layers):
        x = thinker_layer(x, layer_weights(W, l), n_q, n_kv)
    h = rms_norm(x, W["out_norm"])
    return h, W["embed"] @ h[-1]


def prefill(prompts: Sequence[Tuple[np.ndarray, np.ndarray, int]], W: Dict[str, np.ndarray], n_layers: int,
            n_q: int, n_kv: int) -> Tuple[np.ndarray, np.ndarray]:
    """Packed batch (reading T4): concatenated hidden states and one logits row
    per prompt."""
    hs, lg = [], []
    for ids, audio, off in prompts:
        h, g = prefill_prompt(ids, audio, off, W, n_layers, n_q, n_kv)
        hs.append(h)
        lg.append(g)
    return np.concatenate(hs), np.stack(lg)
