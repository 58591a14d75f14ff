"""Seeded synthetic inputs for the Thinker prefill over a spliced prompt.

Random numbers shaped into weight tensors and token-id prompts; none of the
decoder's arithmetic lives here.

Shapes follow the Thinker hyper-parameters on the qwenasr.cpp architecture
page (section "GGUF layout"): 28 layers, 16 query heads and 8 KV heads of
head_dim 128, vocab 151936; hidden / FFN 1024 / 3072 (0.6B) and 2048 / 6144
(1.7B).  ``THINKER_TINY`` is an fp32 miniature for fast parity runs.

Prompts follow the layout of section "Prompt assembly and audio splice":
a text prefix, ``<|audio_start|>``, one placeholder per encoder state,
``<|audio_end|>``, a text suffix.  Text ids are random; the special ids are
the page's where the vocabulary has them.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

from . import round_to_bf16

AUDIO_START, AUDIO_END, AUDIO_PAD = 151669, 151670, 151676   # [qwenasr] "GGUF layout"
PREFIX_LEN, SUFFIX_LEN = 9, 6


@dataclasses.dataclass(frozen=True)
class ThinkerDims:
    """Thinker shape; mirrors the ``qa_thinker_dims`` struct of the C ABI."""
    hidden: int = 2048
    n_layers: int = 28
    n_q_heads: int = 16
    n_kv_heads: int = 8
    head_dim: int = 128
    ffn_dim: int = 6144
    vocab: int = 151936
    dtype: str = "bf16"


THINKER_TINY = ThinkerDims(hidden=256, n_layers=2, n_q_heads=2, n_kv_heads=1, ffn_dim=512, vocab=1000,
                           dtype="f32")
THINKER_06B = ThinkerDims(hidden=1024, n_layers=28, n_q_heads=16, n_kv_heads=8, ffn_dim=3072)
THINKER_17B = ThinkerDims(hidden=2048, n_layers=28, n_q_heads=16, n_kv_heads=8, ffn_dim=6144)

LAYER_FIELDS = ("attn_norm", "q_w", "k_w", "v_w", "q_norm", "k_norm", "o_w", "ffn_norm", "gate_w", "up_w",
                "down_w")


def weight_shapes(d: ThinkerDims):
    """(name, shape) in draw order, PyTorch Linear layout (out, in)."""
    H, F, dq, dkv = d.hidden, d.ffn_dim, d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim
    s = [("embed", (d.vocab, H))]
    for l in range(d.n_layers):
        for f, shp in zip(LAYER_FIELDS, ((H,), (dq, H), (dkv, H), (dkv, H), (d.head_dim,), (d.head_dim,),
                                         (H, dq), (H,), (F, H), (F, H), (H, F))):
            s.append((f"layers.{l}.{f}", shp))
    s.append(("out_norm", (H,)))
    return s


def make_weights(d: ThinkerDims, seed: int, std: float = 0.02) -> Dict[str, np.ndarray]:
    """N(0, std^2) matrices; RMSNorm gains 1 + N(0, std^2); bf16 shapes get
    their values rounded to bf16 (float32 arrays holding bf16 values)."""
    rng = np.random.default_rng(seed)
    w = {}
    for name, shp in weight_shapes(d):
        a = rng.standard_normal(shp, dtype=np.float32) * np.float32(std)
        if name.endswith("norm"):
            a = a + np.float32(1.0)
        if d.dtype == "bf16":
            a = round_to_bf16(a)
        w[name] = a
    return w


def make_prompt(n_audio: int, vocab: int, seed) -> Tuple[np.ndarray, int]:
    """(ids [T] int32, audio_offset): prefix, audio_start, n_audio
    placeholders, audio_end, suffix."""
    rng = np.random.default_rng(seed)
    text_hi = min(vocab, 151643)
    special = (lambda i: i) if vocab > AUDIO_PAD else (lambda i: int(rng.integers(0, vocab)))
    pre = rng.integers(0, text_hi, PREFIX_LEN)
    suf = rng.integers(0, text_hi, SUFFIX_LEN)
    ids = np.concatenate([pre, [special(AUDIO_START)], np.full(n_audio, special(AUDIO_PAD)),
                          [special(AUDIO_END)], suf]).astype(np.int32)
    return ids, PREFIX_LEN + 1


def make_audio_states(n_audio: int, hidden: int, seed) -> np.ndarray:
    """Stand-in encoder states (N(0, 1) rows) for oracle-only tests; the GPU
    tests splice the encoder's real output."""
    return np.random.default_rng(seed).standard_normal((n_audio, hidden)).astype(np.float32)
