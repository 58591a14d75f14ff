"""Seeded synthetic inputs for the AuT audio-encoder forward.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random numbers and shapes them into PCM clips and weight
tensors; it contains none of the encoder's arithmetic (no framing, DFT, mel,
convolution, attention or normalisation).

Workloads (the five shapes the encoder is exercised on):

* ``tiny``   - fp32, one 2 s clip of a 440 Hz tone plus N(0, 0.01) noise,
               conv width 32, d 256, 2 layers, 4 heads, FFN 1024, out 256.
* ``b06_1``  - 0.6B-shaped bf16 encoder (conv 480, d 896, 18 layers, 14 heads,
               FFN 3584, out 1024), one 30 s speech-like clip.
* ``b06_32`` - the same encoder, 32 clips of U(1, 30) s (seed 3).
* ``b17_20m``- 1.7B-shaped bf16 encoder (conv 480, d 1024, 24 layers, 16 heads,
               FFN 4096, out 2048), one 20-minute clip (19.2 M samples).
* ``b17_16`` - the same encoder, 16 clips of log-uniform 10-300 s (seed 5).

The dimensions follow the audio-tower hyper-parameters listed on the
qwenasr.cpp architecture page (section "GGUF layout"): 128 mel bins, conv
width 480, 100-frame chunks, 8 chunks per attention window.

Every array is a pure function of its seed (NumPy PCG64 ``default_rng``).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

SAMPLE_RATE = 16000


@dataclasses.dataclass(frozen=True)
class Dims:
    """Encoder shape; mirrors the ``qa_dims`` struct of the C ABI."""
    n_mels: int = 128
    conv_channels: int = 480
    d_model: int = 1024
    n_layers: int = 24
    n_heads: int = 16
    head_dim: int = 64
    ffn_dim: int = 4096
    output_dim: int = 2048
    chunk_frames: int = 100
    window_chunks: int = 8
    dtype: str = "bf16"          # "f32" or "bf16": weight / operand precision


DIMS_TINY = Dims(conv_channels=32, d_model=256, n_layers=2, n_heads=4, head_dim=64,
                 ffn_dim=1024, output_dim=256, dtype="f32")
DIMS_06B = Dims(conv_channels=480, d_model=896, n_layers=18, n_heads=14, head_dim=64,
                ffn_dim=3584, output_dim=1024, dtype="bf16")
DIMS_17B = Dims(conv_channels=480, d_model=1024, n_layers=24, n_heads=16, head_dim=64,
                ffn_dim=4096, output_dim=2048, dtype="bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    audio_seed: int
    weight_seed: int
    kind: str                     # "tone" | "fixed" | "uniform" | "loguniform"
    n_clips: int
    fixed_len: int = 0            # samples, for kind in ("tone", "fixed")
    lo_s: float = 0.0             # seconds, for the random-length kinds
    hi_s: float = 0.0
    description: str = ""


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", DIMS_TINY, 1, 100, "tone", 1, fixed_len=32000,
                     description="fp32 tiny encoder, one 2 s 440 Hz tone + N(0,0.01) noise"),
    "b06_1": Workload("b06_1", DIMS_06B, 2, 106, "fixed", 1, fixed_len=480000,
                      description="0.6B-shaped bf16 encoder, one 30 s clip"),
    "b06_32": Workload("b06_32", DIMS_06B, 3, 106, "uniform", 32, lo_s=1.0, hi_s=30.0,
                       description="0.6B-shaped bf16 encoder, 32 clips U(1,30) s"),
    "b17_20m": Workload("b17_20m", DIMS_17B, 4, 117, "fixed", 1, fixed_len=19_200_000,
                        description="1.7B-shaped bf16 encoder, one 20-minute clip"),
    "b17_16": Workload("b17_16", DIMS_17B, 5, 117, "loguniform", 16, lo_s=10.0, hi_s=300.0,
                       description="1.7B-shaped bf16 encoder, 16 clips logU(10,300) s"),
}


# ----------------------------------------------------------------------------- audio

def clip_lengths(wl: Workload) -> np.ndarray:
    """Clip lengths in samples (int64)."""
    if wl.kind in ("tone", "fixed"):
        return np.full(wl.n_clips, wl.fixed_len, dtype=np.int64)
    rng = np.random.default_rng(wl.audio_seed)
    if wl.kind == "uniform":
        sec = rng.uniform(wl.lo_s, wl.hi_s, wl.n_clips)
    elif wl.kind == "loguniform":
        sec = np.exp(rng.uniform(np.log(wl.lo_s), np.log(wl.hi_s), wl.n_clips))
    else:
        raise ValueError(wl.kind)
    return np.rint(sec * SAMPLE_RATE).astype(np.int64)


def tone_clip(n: int, seed_seq, freq: float = 440.0, amp: float = 0.3,
              noise_std: float = 0.01) -> np.ndarray:
    """amp*sin(2*pi*freq*t) + N(0, noise_std^2), float32."""
    rng = np.random.default_rng(seed_seq)
    t = np.arange(n, dtype=np.float64) / SAMPLE_RATE
    x = amp * np.sin(2.0 * np.pi * freq * t) + noise_std * rng.standard_normal(n)
    return x.astype(np.float32)


def speech_like_clip(n: int, seed_seq) -> np.ndarray:
    """0.05-rms pink noise plus three amplitude-modulated tones, float32.

    Pink noise: white N(0,1) shaped by 1/sqrt(f) in the real-FFT domain with the
    DC bin zeroed, rescaled to rms 0.05.  Tones: carrier U(200, 3400) Hz,
    modulator U(2, 8) Hz (a syllabic rate), 0.1*(1+0.8 sin(2 pi fm t + p1))
    * sin(2 pi fc t + p2) with phases U(0, 2 pi).  The result spans well over
    60 dB between loud tone bins and quiet noise bins.
    """
    if n == 0:
        return np.zeros(0, dtype=np.float32)
    rng = np.random.default_rng(seed_seq)
    white = rng.standard_normal(n)
    spec = np.fft.rfft(white)
    f = np.arange(spec.shape[0], dtype=np.float64)
    shape = np.zeros_like(f)
    shape[1:] = 1.0 / np.sqrt(f[1:])
    pink = np.fft.irfft(spec * shape, n=n)
    pink *= 0.05 / max(np.sqrt(np.mean(pink * pink)), 1e-30)
    t = np.arange(n, dtype=np.float64) / SAMPLE_RATE
    x = pink
    for _ in range(3):
        fc = rng.uniform(200.0, 3400.0)
        fm = rng.uniform(2.0, 8.0)
        p1, p2 = rng.uniform(0.0, 2.0 * np.pi, 2)
        x = x + 0.1 * (1.0 + 0.8 * np.sin(2 * np.pi * fm * t + p1)) * np.sin(2 * np.pi * fc * t + p2)
    return x.astype(np.float32)


def make_audio(wl: Workload) -> List[np.ndarray]:
    """One float32 array per clip, in clip order."""
    out = []
    for i, n in enumerate(clip_lengths(wl)):
        if wl.kind == "tone":
            out.append(tone_clip(int(n), [wl.audio_seed, i]))
        else:
            out.append(speech_like_clip(int(n), [wl.audio_seed, i]))
    return out


# ----------------------------------------------------------------------------- weights

LAYER_FIELDS = ("ln1_w", "ln1_b", "q_w", "q_b", "k_w", "k_b", "v_w", "v_b", "o_w", "o_b",
                "ln2_w", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")


def weight_shapes(d: Dims):
    """(name, shape) in draw order; PyTorch layouts: Linear (out, in), conv
    (C_out, C_in, k_mel, k_time).  ``conv_out`` is a Linear without bias whose
    input index is c*16 + f (channel outer, frequency inner)."""
    C, D, F, O = d.conv_channels, d.d_model, d.ffn_dim, d.output_dim
    fq = d.n_mels // 8
    s = [("conv1_w", (C, 1, 3, 3)), ("conv1_b", (C,)),
         ("conv2_w", (C, C, 3, 3)), ("conv2_b", (C,)),
         ("conv3_w", (C, C, 3, 3)), ("conv3_b", (C,)),
         ("conv_out_w", (D, C * fq))]
    for l in range(d.n_layers):
        for f, shp in zip(LAYER_FIELDS, ((D,), (D,), (D, D), (D,), (D, D), (D,), (D, D), (D,),
                                         (D, D), (D,), (D,), (D,), (F, D), (F,), (D, F), (D,))):
            s.append((f"layers.{l}.{f}", shp))
    s += [("post_ln_w", (D,)), ("post_ln_b", (D,)),
          ("proj1_w", (D, D)), ("proj1_b", (D,)),
          ("proj2_w", (O, D)), ("proj2_b", (O,))]
    return s


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 arrays holding exactly representable bf16 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-representable")
    return (u >> 16).astype(np.uint16)


def make_weights(d: Dims, seed: int, std: float = 0.02) -> Dict[str, np.ndarray]:
    """Random-init weights: N(0, std^2) for matrices and biases, LayerNorm
    gamma = 1 + N(0, std^2), beta = N(0, std^2).  bf16 encoders get their
    values rounded to bf16 (stored as float32 holding bf16 values)."""
    rng = np.random.default_rng(seed)
    w = {}
    for name, shp in weight_shapes(d):
        a = rng.standard_normal(shp, dtype=np.float32) * np.float32(std)
        if name.endswith(("ln1_w", "ln2_w", "post_ln_w")):
            a = a + np.float32(1.0)
        if d.dtype == "bf16":
            a = round_to_bf16(a)
        w[name] = a
    return w

