"""fp64 NumPy oracle of the AuT audio-encoder forward (test infrastructure only).

Each function names the passage it follows.  Page short names:
[OneSpeech] "Front end and graph numerics"; [qwenasr] qwenasr.cpp architecture
page; [M*] the M* ASR page, Qwen3-ASR "Graph" paragraph.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf

SAMPLE_RATE = 16000
N_FFT = 400
HOP = 160
N_MELS = 128
F_MAX = 8000.0
LN_EPS = 1e-5            # not stated on the pages; PyTorch LayerNorm default
MAX_SAMPLES = 20 * 60 * SAMPLE_RATE   # [M*]: a request hears up to 20 minutes
MAX_FULL_INPUT = 30 * SAMPLE_RATE     # [OneSpeech]: longer inputs are chunked before recognition


class InvalidInput(ValueError):
    """An input the input contract rejects ([OneSpeech] "Low-level recognition")."""


# ------------------------------------------------------------------- front end

def hann_periodic(n: int = N_FFT) -> np.ndarray:
    """Periodic Hann window w[i] = 0.5 - 0.5 cos(2 pi i / n) ([OneSpeech]
    "400-sample periodic Hann windows")."""
    i = np.arange(n, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * i / n)


def reflect_pad(x: np.ndarray, p: int) -> np.ndarray:
    """Mirror padding without repeating the edge sample: x[-i] = x[i]
    ([OneSpeech] "centered reflection"; [qwenasr] "Mel frontend": reflect pad by
    n_fft/2).  Needs len(x) > p."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[0] <= p:
        raise InvalidInput("reflection padding needs more than %d samples" % p)
    left = x[1:p + 1][::-1]
    right = x[-p - 1:-1][::-1]
    return np.concatenate([left, x, right])


def stft_frames(x: np.ndarray, n_fft: int = N_FFT, hop: int = HOP) -> np.ndarray:
    """All centered frames: frame j = xp[hop*j : hop*j + n_fft] for
    j = 0 .. floor(len/hop) (the final one is dropped later)."""
    xp = reflect_pad(x, n_fft // 2)
    n_frames = 1 + (xp.shape[0] - n_fft) // hop
    idx = hop * np.arange(n_frames)[:, None] + np.arange(n_fft)[None, :]
    return xp[idx]


def dft_matrices(n_fft: int = N_FFT) -> Tuple[np.ndarray, np.ndarray]:
    """cos / sin DFT bases, [n_fft, n_fft//2 + 1], trig in fp64 ([qwenasr]
    "Mel DFT without an FFT op": the transform is two real matmuls against
    precomputed cos and sin matrices)."""
    nn = np.arange(n_fft, dtype=np.float64)[:, None]
    k = np.arange(n_fft // 2 + 1, dtype=np.float64)[None, :]
    ang = 2.0 * np.pi * ((nn * k) % n_fft) / n_fft
    return np.cos(ang), np.sin(ang)


def power_spectrum(frames: np.ndarray, window: Optional[np.ndarray] = None) -> np.ndarray:
    """|X_k|^2 = Re^2 + Im^2 with X_k = sum_n w[n] fr[n] e^{-2 pi i k n / N}
    ([qwenasr] "Mel frontend": magnitude squared, no sqrt)."""
    n_fft = frames.shape[-1]
    if window is None:
        window = hann_periodic(n_fft)
    fw = frames * window[None, :]
    c, s = dft_matrices(n_fft)
    re = fw @ c
    im = -(fw @ s)
    return re * re + im * im


def hz_to_mel(f):
    """Slaney's Auditory-Toolbox mel scale (librosa htk=False): linear 3f/200
    below 1 kHz, logarithmic above with 27 mels per factor 6.4 ([qwenasr]
    "Glossary": Slaney mel)."""
    f = np.asarray(f, dtype=np.float64)
    lin = 3.0 * f / 200.0
    log = 15.0 + 27.0 * np.log(np.maximum(f, 1e-300) / 1000.0) / np.log(6.4)
    return np.where(f >= 1000.0, log, lin)


def mel_to_hz(m):
    m = np.asarray(m, dtype=np.float64)
    lin = 200.0 * m / 3.0
    log = 1000.0 * np.exp((m - 15.0) * np.log(6.4) / 27.0)
    return np.where(m >= 15.0, log, lin)


def mel_filterbank(n_mels: int = N_MELS, n_fft: int = N_FFT, sr: int = SAMPLE_RATE,
                   fmin: float = 0.0, fmax: float = F_MAX) -> np.ndarray:
    """Slaney-scale, area-normalised triangular filters [n_mels, n_fft//2+1]
    ([OneSpeech] "Slaney mel filters"; [qwenasr] "Mel frontend" fmin 0,
    fmax 8000).  Edges: n_mels+2 points uniform in mel; filter m rises from
    edge m to m+1, falls to m+2, scaled by 2/(f_{m+2} - f_m)."""
    freqs = np.arange(n_fft // 2 + 1, dtype=np.float64) * sr / n_fft
    edges = mel_to_hz(np.linspace(hz_to_mel(fmin), hz_to_mel(fmax), n_mels + 2))
    fb = np.zeros((n_mels, freqs.shape[0]))
    for m in range(n_mels):
        lo, ce, hi = edges[m], edges[m + 1], edges[m + 2]
        up = (freqs - lo) / (ce - lo)
        down = (hi - freqs) / (hi - ce)
        fb[m] = np.maximum(0.0, np.minimum(up, down)) * (2.0 / (hi - lo))
    return fb


F32_MAX = float(np.finfo(np.float32).max)


def log_mel_raw(x: np.ndarray) -> np.ndarray:
    """log10(max(mel energy, 1e-10)) for the kept frames, [n_mels, F] with
    F = floor(len/160) ([qwenasr] "Mel frontend": clamp then log; the trailing
    STFT frame is dropped; [OneSpeech] "power floor 1e-10").

    Only the lower bound applies.  [qwenasr] "Mel frontend" also caps the mel
    energy at 1e30 before the log; [OneSpeech] "Front end and graph numerics"
    names only the 1e-10 floor and holds its features to the published float32
    Whisper extractor, which has no cap, and "Low-level recognition" rejects
    inputs whose power leaves the float32 range instead.  So energies in
    (1e30, float32 max] keep their logarithm (above 30).

    Raises InvalidInput for a nonfinite sample or a power / mel value beyond
    float32 range ([OneSpeech] "Low-level recognition": such inputs are
    rejected).  The check covers every sample and every frame, including the
    final STFT frame that is dropped from the output."""
    if not np.all(np.isfinite(x)):
        raise InvalidInput("nonfinite sample")
    fr = stft_frames(x)
    p = power_spectrum(fr)                 # [F+1, 201]
    e = p @ mel_filterbank().T             # [F+1, 128]
    if p.max(initial=0.0) > F32_MAX or e.max(initial=0.0) > F32_MAX:
        raise InvalidInput("power beyond float32 range")
    lg = np.log10(np.maximum(e, 1e-10))
    return lg[:-1].T                       # drop the last frame, mel-major


def log_mel(x: np.ndarray) -> np.ndarray:
    """Normalised log-mel [128, F]: (max(l, max(l) - 8) + 4) / 4 with the max
    taken over this clip's kept frames ([OneSpeech] "log10 peak-minus-eight
    clipping, then (x + 4) / 4"; [qwenasr] "Mel frontend" host tail)."""
    lg = log_mel_raw(x)
    if lg.shape[1] == 0:
        return lg
    return (np.maximum(lg, lg.max() - 8.0) + 4.0) / 4.0


# ------------------------------------------------------------------- planner

def after_cnn_len(m: int) -> int:
    """Length after the three stride-2 convolutions: ceil-halve three times
    ([qwenasr] "Conv2d subsampling stem", after-cnn length)."""
    for _ in range(3):
        m = (m - 1) // 2 + 1
    return m


def validate_clip(n: int) -> None:
    """[OneSpeech] "Low-level recognition": empty is allowed, nonempty input
    must exceed 200 samples; [M*]: at most 20 minutes per request."""
    if n < 0:
        raise InvalidInput("negative length")
    if 0 < n <= 200:
        raise InvalidInput("nonempty audio must exceed 200 samples")
    if n > MAX_SAMPLES:
        raise InvalidInput("clip longer than 20 minutes")


def chunk_lengths(n_frames: int, chunk: int = 100) -> List[int]:
    """Consecutive chunks of `chunk` frames from frame 0; the tail keeps the
    remainder ([OneSpeech] "Convolution chunks have 100 mel frames")."""
    out = [chunk] * (n_frames // chunk)
    if n_frames % chunk:
        out.append(n_frames % chunk)
    return out


def clip_num_tokens(n_samples: int, chunk: int = 100) -> int:
    if n_samples == 0:
        return 0
    return sum(after_cnn_len(m) for m in chunk_lengths(n_samples // HOP, chunk))


def window_bounds(n_tokens: int, window: int = 104) -> List[Tuple[int, int]]:
    """Consecutive attention windows of a clip's tokens ([qwenasr] "Windowed
    audio tower": 13 * 8 = 104 after-cnn frames; [M*]: one segment per window
    of every request)."""
    return [(s, min(s + window, n_tokens)) for s in range(0, n_tokens, window)]


# ------------------------------------------------------------------- stem

def gelu(z: np.ndarray) -> np.ndarray:
    """Exact erf GELU z * (1 + erf(z / sqrt 2)) / 2 ([qwenasr] "Conv2d stem":
    gelu_erf, not the tanh approximation)."""
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def conv2d_k3s2p1(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """z[co,i,j] = b[co] + sum_{ci,a,b} w[co,ci,a,b] x[ci, 2i+a-1, 2j+b-1],
    zero outside the input; x [Cin, H, W] -> [Cout, ceil(H/2), ceil(W/2)]
    ([qwenasr] "Conv2d subsampling stem": conv2d kernel 3, stride 2, padding 1;
    "Conv2d stem": im2col plus matmul)."""
    cin, h, wd = x.shape
    ho, wo = (h - 1) // 2 + 1, (wd - 1) // 2 + 1
    xp = np.zeros((cin, h + 2, wd + 2))
    xp[:, 1:h + 1, 1:wd + 1] = x
    cols = np.empty((cin, 3, 3, ho, wo))
    for a in range(3):
        for bb in range(3):
            cols[:, a, bb] = xp[:, a:a + 2 * ho:2, bb:bb + 2 * wo:2]
    cout = w.shape[0]
    z = w.reshape(cout, cin * 9) @ cols.reshape(cin * 9, ho * wo)
    return z.reshape(cout, ho, wo) + b[:, None, None]


def stem_chunk(mel_chunk: np.ndarray, W: Dict[str, np.ndarray], n_valid: int,
               tail: str = "A") -> np.ndarray:
    """Conv stem on one chunk of normalised log-mel [128, m], m <= 100; returns
    the pre-PE tokens [after_cnn_len(m), d] ([qwenasr] "Conv2d subsampling
    stem": 3 x (conv + bias + gelu), permute to channel-outer /
    frequency-inner, reshape to C*16, conv_out Linear without bias).

    tail="A": the chunk is zero-padded to 100 frames before the stem and only
    the first after_cnn_len(m) rows are kept ([OneSpeech]: chunks "padded
    independently").  tail="B": the stem runs on the m frames as they are.
    """
    m = mel_chunk.shape[1]
    assert m == n_valid
    if tail == "A" and m < 100:
        img = np.zeros((mel_chunk.shape[0], 100))
        img[:, :m] = mel_chunk
    else:
        img = mel_chunk
    z = img[None].astype(np.float64)
    for l in (1, 2, 3):
        z = gelu(conv2d_k3s2p1(z, W[f"conv{l}_w"], W[f"conv{l}_b"]))
    c, f, t = z.shape                      # [C, 16, t]
    v = z.transpose(2, 0, 1).reshape(t, c * f)   # index c*16 + f
    tok = v @ W["conv_out_w"].T
    return tok[:after_cnn_len(m)]


def sinusoid_pe(n_pos: int, d: int) -> np.ndarray:
    """pe[t, i] = sin(t inv_i), pe[t, d/2 + i] = cos(t inv_i),
    inv_i = exp(-ln(10000) i / (d/2 - 1)) ([qwenasr] "Windowed audio tower")."""
    half = d // 2
    inv = np.exp(-math.log(10000.0) / (half - 1) * np.arange(half, dtype=np.float64))
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.sin(ang), np.cos(ang)], axis=1)


# ------------------------------------------------------------------- encoder

def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm with bias over the last axis ([qwenasr] "Windowed audio
    tower": LayerNorm with bias)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def softmax(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def mha(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int) -> np.ndarray:
    """Bidirectional multi-head attention over one segment, scale 1/sqrt(hd),
    no RoPE ([qwenasr] "Windowed audio tower", "Attention and RoPE")."""
    t, d = q.shape
    hd = d // n_heads
    out = np.empty_like(q)
    for h in range(n_heads):
        sl = slice(h * hd, (h + 1) * hd)
        a = softmax(q[:, sl] @ k[:, sl].T / math.sqrt(hd))
        out[:, sl] = a @ v[:, sl]
    return out


def encoder_layer(x: np.ndarray, L: Dict[str, np.ndarray], segments: Sequence[Tuple[int, int]],
                  n_heads: int) -> np.ndarray:
    """Pre-norm block: x += O(attn(LN1 x)); x += FC2(gelu(FC1(LN2 x)))
    ([qwenasr] "Windowed audio tower"; bias on q/k/v/o and the FFN).
    Attention runs separately inside each [s, e) segment (block-diagonal)."""
    h = layer_norm(x, L["ln1_w"], L["ln1_b"])
    q = h @ L["q_w"].T + L["q_b"]
    k = h @ L["k_w"].T + L["k_b"]
    v = h @ L["v_w"].T + L["v_b"]
    o = np.empty_like(q)
    for s, e in segments:
        o[s:e] = mha(q[s:e], k[s:e], v[s:e], n_heads)
    x = x + o @ L["o_w"].T + L["o_b"]
    h = layer_norm(x, L["ln2_w"], L["ln2_b"])
    u = gelu(h @ L["fc1_w"].T + L["fc1_b"])
    return x + u @ L["fc2_w"].T + L["fc2_b"]


def output_head(x: np.ndarray, W: Dict[str, np.ndarray]) -> np.ndarray:
    """post_norm LayerNorm, proj1 (d -> d), gelu, proj2 (d -> output_dim)
    ([qwenasr] "Windowed audio tower")."""
    h = layer_norm(x, W["post_ln_w"], W["post_ln_b"])
    u = gelu(h @ W["proj1_w"].T + W["proj1_b"])
    return u @ W["proj2_w"].T + W["proj2_b"]


def layer_weights(W: Dict[str, np.ndarray], l: int) -> Dict[str, np.ndarray]:
    pre = f"layers.{l}."
    return {k[len(pre):]: v for k, v in W.items() if k.startswith(pre)}


def as_f64(W: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """Expand weights exactly to fp64 ([OneSpeech]: Binary32 expands the
    bfloat16 tensors exactly)."""
    return {k: np.asarray(v, dtype=np.float64) for k, v in W.items()}


# ------------------------------------------------------------------- forward

def encode_clip(x: np.ndarray, W: Dict[str, np.ndarray], n_layers: int, n_heads: int,
                chunk: int = 100, window_chunks: int = 8,
                windows: Optional[Sequence[int]] = None, tail: str = "A",
                taps: Optional[dict] = None, mel: Optional[np.ndarray] = None) -> Dict[int, np.ndarray]:
    """Forward of one clip.  Returns {window index: output rows [w, out]}.

    window_chunks = 0 selects full-input attention: the whole clip (at most
    30 s) is one attention segment ([OneSpeech] "Front end and graph
    numerics": the CPU graphs attend over the whole bounded input).

    The front end runs over the whole clip (its max normalises every frame);
    after it, chunks never mix and attention never crosses a window, so a
    window's rows depend only on its own 8 chunks.  `windows` selects which
    windows to compute (all if None) -- the definition restricted to them.
    `mel` is this clip's log_mel(x) when the caller already has it (several
    calls over disjoint windows of one clip then share it).
    """
    validate_clip(x.shape[0])
    if window_chunks == 0 and x.shape[0] > MAX_FULL_INPUT:
        raise InvalidInput("full-input attention takes clips of at most 30 s")
    if x.shape[0] == 0:
        return {}
    if mel is None:
        mel = log_mel(x)
    if taps is not None:
        taps["log_mel"] = mel
    lens = chunk_lengths(mel.shape[1], chunk)
    offs = np.concatenate([[0], np.cumsum(lens)])
    per_chunk = [after_cnn_len(m) for m in lens]
    n_tok = sum(per_chunk)
    if window_chunks == 0:            # full-input attention: one segment per clip
        wb, per_win = [(0, n_tok)], len(lens)
    else:
        wb, per_win = window_bounds(n_tok, after_cnn_len(chunk) * window_chunks), window_chunks
    sel = range(len(wb)) if windows is None else windows
    out = {}
    for wi in sel:
        c0, c1 = wi * per_win, min((wi + 1) * per_win, len(lens))
        rows, pre_pe = [], []
        for c in range(c0, c1):
            t = stem_chunk(mel[:, offs[c]:offs[c + 1]], W, lens[c], tail)
            pre_pe.append(t)
            rows.append(t + sinusoid_pe(t.shape[0], t.shape[1]))
        x0 = np.concatenate(rows, axis=0)
        assert x0.shape[0] == wb[wi][1] - wb[wi][0]
        seg = [(0, x0.shape[0])]
        h = x0
        for l in range(n_layers):
            h = encoder_layer(h, layer_weights(W, l), seg, n_heads)
            if taps is not None and l == 0:
                taps.setdefault("layer0", {})[wi] = h
        out[wi] = output_head(h, W)
        if taps is not None:
            taps.setdefault("stem", {})[wi] = np.concatenate(pre_pe, axis=0)
    return out


def encode(pcm: Sequence[np.ndarray], W: Dict[str, np.ndarray], n_layers: int, n_heads: int,
           chunk: int = 100, window_chunks: int = 8, tail: str = "A") -> np.ndarray:
    """Whole packed batch: rows clip-major, then chunk, then token-in-chunk
    ([M*]: one packed forward, one attention segment per window of every
    request).  Returns [sum tokens, output_dim]."""
    Wd = as_f64(W)
    parts = []
    for x in pcm:
        res = encode_clip(np.asarray(x), Wd, n_layers, n_heads, chunk, window_chunks, tail=tail)
        parts.extend(res[i] for i in sorted(res))
    if not parts:
        return np.zeros((0, W["proj2_w"].shape[0]))
    return np.concatenate(parts, axis=0)
