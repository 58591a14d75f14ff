"""Error model of the bf16 operand policy for the Thinker prefill (test
helper, not the oracle): the oracle's forward with every value that the GPU
path stores as bf16 rounded to bf16 (nearest even) at the same operator
boundaries, everything else in fp64.  Comparing it with the exact oracle shows
how far the policy alone moves the result, which is what the bf16 tolerance of
the parity test is set against; comparing it with the GPU shows that the GPU
applies the policy and nothing else."""
from __future__ import annotations

import numpy as np

import oracle.thinker as TH


def bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), via float32."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def _attention(q, k, v):
    """Causal GQA with the probabilities rounded to bf16 for P.V and the
    normalisation by the unrounded sum, as the kernel does."""
    T, hq, d = q.shape
    group = hq // k.shape[1]
    out = np.empty_like(q)
    mask = np.tril(np.ones((T, T), dtype=bool))
    for h in range(hq):
        s = q[:, h] @ k[:, h // group].T / np.sqrt(d)
        s = np.where(mask, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h] = (bf16(p) @ v[:, h // group]) / p.sum(axis=1, keepdims=True)
    return out


def prefill_prompt(ids, audio, audio_offset, W, n_layers, n_q, n_kv):
    x = TH.splice(ids, audio, audio_offset, W["embed"])
    T = x.shape[0]
    d = TH.HEAD_DIM
    pos = np.arange(T)
    for l in range(n_layers):
        L = TH.layer_weights(W, l)
        a = bf16(TH.rms_norm(x, L["attn_norm"]))
        q = bf16(a @ L["q_w"].T).reshape(T, n_q, d)
        k = bf16(a @ L["k_w"].T).reshape(T, n_kv, d)
        v = bf16(a @ L["v_w"].T).reshape(T, n_kv, d)
        q = bf16(TH.rope_neox(TH.rms_norm(q, L["q_norm"]), pos))
        k = bf16(TH.rope_neox(TH.rms_norm(k, L["k_norm"]), pos))
        o = bf16(_attention(q, k, v)).reshape(T, n_q * d)
        x = x + o @ L["o_w"].T
        a = bf16(TH.rms_norm(x, L["ffn_norm"]))
        x = x + bf16(TH.silu(a @ L["gate_w"].T) * (a @ L["up_w"].T)) @ L["down_w"].T
    h = TH.rms_norm(x, W["out_norm"])
    return h, W["embed"] @ bf16(h[-1])
