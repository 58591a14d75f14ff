"""ctypes binding of libqa_encoder.so, with the C ABI's names.

Argument marshalling only: every step of the encoder runs in the HIP library.
If the library is missing, importing this module raises -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Mapping, Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqa_encoder.so")

QA_ABI_VERSION = 1
QA_STATUS_OK = 0
QA_STATUS_INVALID_PARAMS = -1
QA_STATUS_LOAD_FAILED = -2
QA_STATUS_ENCODE_FAILED = -3
QA_STATUS_OOM = -4
QA_DTYPE_F32 = 0
QA_DTYPE_BF16 = 1
QA_TAP_LOG_MEL = 0
QA_TAP_STEM = 1
QA_TAP_LAYER0 = 2
QA_NOALLOC_SCRATCH_BYTES = 160 * 1024 * 1024

EXPORTS = ("qa_abi_version", "qa_last_error", "qa_encode_num_tokens", "qa_encoder_create",
           "qa_encoder_set_stream", "qa_encoder_set_max_lanes", "qa_encode", "qa_encode_noalloc", "qa_encoder_enable_taps", "qa_encoder_tap",
           "qa_encoder_set_profiling", "qa_encoder_kernel_times", "qa_encoder_set_profiling_label",
           "qa_encoder_free", "qa_resample_length", "qa_resampler_create", "qa_resample", "qa_resampler_free",
           "qa_thinker_create", "qa_thinker_set_stream", "qa_thinker_prefill", "qa_thinker_free")


class qa_dims(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("abi_version", "n_mels", "conv_channels", "d_model", "n_layers",
                                       "n_heads", "head_dim", "ffn_dim", "output_dim", "chunk_frames",
                                       "window_chunks", "dtype")]


_VP = C.c_void_p
_VPP = C.POINTER(C.c_void_p)


class qa_weights(C.Structure):
    _fields_ = ([(n, _VP) for n in ("conv1_w", "conv1_b", "conv2_w", "conv2_b", "conv3_w", "conv3_b",
                                    "conv_out_w")]
                + [(n, _VPP) for n in ("ln1_w", "ln1_b", "q_w", "q_b", "k_w", "k_b", "v_w", "v_b",
                                       "o_w", "o_b", "ln2_w", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")]
                + [(n, _VP) for n in ("post_ln_w", "post_ln_b", "proj1_w", "proj1_b", "proj2_w", "proj2_b")])


class qa_thinker_dims(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("abi_version", "hidden", "n_layers", "n_q_heads", "n_kv_heads", "head_dim",
                                       "ffn_dim", "vocab", "dtype")]


THINKER_LAYER_FIELDS = ("attn_norm", "q_w", "k_w", "v_w", "q_norm", "k_norm", "o_w", "ffn_norm", "gate_w", "up_w",
                        "down_w")


class qa_thinker_weights(C.Structure):
    _fields_ = [("embed", _VP)] + [(n, _VPP) for n in THINKER_LAYER_FIELDS] + [("out_norm", _VP)]


class QAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


def _load() -> C.CDLL:
    # PyTorch ships its own HIP runtime (SONAME libamdhip64.so.7); loading
    # torch first makes the library bind to that same runtime instead of a
    # second copy, so torch's device pointers and streams are valid here.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run audio_encoder_front_amd.build.build()")
    lib = C.CDLL(LIB_PATH)
    lib.qa_abi_version.restype = C.c_int
    lib.qa_last_error.restype = C.c_char_p
    lib.qa_encode_num_tokens.restype = C.c_int64
    lib.qa_encode_num_tokens.argtypes = [C.c_int64]
    lib.qa_encoder_create.restype = C.c_void_p
    lib.qa_encoder_create.argtypes = [C.POINTER(qa_weights), C.POINTER(qa_dims)]
    lib.qa_encoder_set_stream.restype = C.c_int
    lib.qa_encoder_set_stream.argtypes = [C.c_void_p, C.c_void_p]
    lib.qa_encode.restype = C.c_int
    lib.qa_encode.argtypes = [C.c_void_p, C.c_void_p, C.POINTER(C.c_int64), C.c_int, C.c_void_p]
    lib.qa_encode_noalloc.restype = C.c_int
    lib.qa_encode_noalloc.argtypes = [C.c_void_p, C.c_void_p, C.POINTER(C.c_int64), C.c_int, C.c_void_p]
    lib.qa_encoder_enable_taps.restype = C.c_int
    lib.qa_encoder_enable_taps.argtypes = [C.c_void_p, C.c_int]
    lib.qa_encoder_tap.restype = C.c_int64
    lib.qa_encoder_tap.argtypes = [C.c_void_p, C.c_int, C.c_void_p, C.c_int64]
    lib.qa_encoder_set_profiling.restype = C.c_int
    lib.qa_encoder_set_profiling.argtypes = [C.c_void_p, C.c_int]
    lib.qa_encoder_set_max_lanes.restype = C.c_int
    lib.qa_encoder_set_max_lanes.argtypes = [C.c_void_p, C.c_int]
    lib.qa_encoder_set_profiling_label.restype = C.c_int
    lib.qa_encoder_set_profiling_label.argtypes = [C.c_void_p, C.c_char_p]
    lib.qa_encoder_kernel_times.restype = C.c_int
    lib.qa_encoder_kernel_times.argtypes = [C.c_void_p, C.POINTER(C.c_char_p), C.POINTER(C.c_double),
                                            C.POINTER(C.c_int64), C.c_int]
    lib.qa_encoder_free.restype = None
    lib.qa_encoder_free.argtypes = [C.c_void_p]
    lib.qa_thinker_create.restype = C.c_void_p
    lib.qa_thinker_create.argtypes = [C.POINTER(qa_thinker_weights), C.POINTER(qa_thinker_dims)]
    lib.qa_thinker_set_stream.restype = C.c_int
    lib.qa_thinker_set_stream.argtypes = [C.c_void_p, C.c_void_p]
    lib.qa_thinker_prefill.restype = C.c_int
    lib.qa_thinker_prefill.argtypes = [C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_int64), C.c_int, C.c_void_p,
                                       C.POINTER(C.c_int64), C.POINTER(C.c_int64), C.c_void_p, C.c_void_p]
    lib.qa_thinker_free.restype = None
    lib.qa_thinker_free.argtypes = [C.c_void_p]
    lib.qa_resample_length.restype = C.c_int64
    lib.qa_resample_length.argtypes = [C.c_int64, C.c_int]
    lib.qa_resampler_create.restype = C.c_void_p
    lib.qa_resampler_create.argtypes = [C.c_int]
    lib.qa_resample.restype = C.c_int
    lib.qa_resample.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]
    lib.qa_resampler_free.restype = None
    lib.qa_resampler_free.argtypes = [C.c_void_p]
    return lib


_lib = _load()


def library() -> C.CDLL:
    return _lib


def qa_abi_version() -> int:
    return _lib.qa_abi_version()


def qa_last_error() -> str:
    return _lib.qa_last_error().decode()


def qa_encode_num_tokens(n_samples: int) -> int:
    return _lib.qa_encode_num_tokens(int(n_samples))


def _check(status: int) -> None:
    if status != QA_STATUS_OK:
        raise QAError(status, qa_last_error())


class Encoder:
    """Owns a qa_encoder handle."""

    def __init__(self, handle: int, dims: qa_dims):
        self.handle = handle
        self.dims = dims

    def __del__(self):
        self.free()

    def free(self):
        if getattr(self, "handle", None):
            _lib.qa_encoder_free(self.handle)
            self.handle = None


def make_dims(d) -> qa_dims:
    """qa_dims from any object/mapping with the Dims fields (dtype 'f32'/'bf16')."""
    get = (lambda k: d[k]) if isinstance(d, Mapping) else (lambda k: getattr(d, k))
    dt = get("dtype")
    dt = {"f32": QA_DTYPE_F32, "bf16": QA_DTYPE_BF16}.get(dt, dt)
    return qa_dims(QA_ABI_VERSION, get("n_mels"), get("conv_channels"), get("d_model"), get("n_layers"),
                   get("n_heads"), get("head_dim"), get("ffn_dim"), get("output_dim"), get("chunk_frames"),
                   get("window_chunks"), int(dt))


def _host_buffer(a: np.ndarray, dtype: int) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == QA_DTYPE_F32:
        return a
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("bf16 weights must hold bf16-representable values")
    return (u >> 16).astype(np.uint16)


def qa_encoder_create(weights: Dict[str, np.ndarray], dims) -> Encoder:
    """weights: name -> array in PyTorch layout (names as in the qa_weights
    struct; per-layer tensors as 'layers.<l>.<name>')."""
    qd = make_dims(dims)
    keep = []

    def ptr(name):
        b = _host_buffer(weights[name], qd.dtype)
        keep.append(b)
        return b.ctypes.data_as(C.c_void_p)

    w = qa_weights()
    for n in ("conv1_w", "conv1_b", "conv2_w", "conv2_b", "conv3_w", "conv3_b", "conv_out_w",
              "post_ln_w", "post_ln_b", "proj1_w", "proj1_b", "proj2_w", "proj2_b"):
        setattr(w, n, ptr(n))
    L = qd.n_layers
    for n in ("ln1_w", "ln1_b", "q_w", "q_b", "k_w", "k_b", "v_w", "v_b", "o_w", "o_b", "ln2_w", "ln2_b",
              "fc1_w", "fc1_b", "fc2_w", "fc2_b"):
        arr = (C.c_void_p * max(L, 1))(*[ptr(f"layers.{l}.{n}") for l in range(L)])
        keep.append(arr)
        setattr(w, n, C.cast(arr, _VPP))
    h = _lib.qa_encoder_create(C.byref(w), C.byref(qd))
    if not h:
        raise QAError(QA_STATUS_LOAD_FAILED, qa_last_error())
    return Encoder(h, qd)


def qa_encoder_set_stream(enc: Encoder, stream) -> None:
    """stream: a torch.cuda.Stream, a raw hipStream_t int, or None."""
    raw = getattr(stream, "cuda_stream", stream)
    _check(_lib.qa_encoder_set_stream(enc.handle, C.c_void_p(raw or 0)))


def qa_encode(enc: Encoder, pcm, lengths: Sequence[int], out) -> None:
    """pcm: device float32 tensor (all clips concatenated); lengths: host
    sequence of int; out: device float32 tensor [total_tokens, output_dim]."""
    _encode_call(_lib.qa_encode, enc, pcm, lengths, out)


def qa_encode_noalloc(enc: Encoder, pcm, lengths: Sequence[int], out) -> None:
    """qa_encode on the library's fixed per-GPU scratch array (no allocation;
    batches up to QA_NOALLOC_SCRATCH_BYTES of workspace; calls on one GPU
    must not overlap)."""
    _encode_call(_lib.qa_encode_noalloc, enc, pcm, lengths, out)


def _encode_call(fn, enc: Encoder, pcm, lengths: Sequence[int], out) -> None:
    n = len(lengths)
    total = sum(int(x) for x in lengths)
    rows = 0
    for x in lengths:
        t = qa_encode_num_tokens(int(x))
        if t < 0:
            raise QAError(QA_STATUS_INVALID_PARAMS, qa_last_error())
        rows += t
    for name, t, need in (("pcm", pcm, total), ("out", out, rows * enc.dims.output_dim)):
        if need == 0:
            continue
        if t is None or not t.is_cuda or t.dtype.itemsize != 4 or not t.dtype.is_floating_point \
                or not t.is_contiguous() or t.numel() < need:
            raise QAError(QA_STATUS_INVALID_PARAMS,
                          f"{name} must be a contiguous float32 device tensor of at least {need} elements")
    arr = (C.c_int64 * max(n, 1))(*[int(x) for x in lengths])
    pp = C.c_void_p(pcm.data_ptr() if pcm is not None and pcm.numel() else 0)
    op = C.c_void_p(out.data_ptr() if out is not None and out.numel() else 0)
    _check(fn(enc.handle, pp, arr, n, op))


def qa_encoder_enable_taps(enc: Encoder, enable: bool) -> None:
    _check(_lib.qa_encoder_enable_taps(enc.handle, 1 if enable else 0))


def qa_encoder_tap(enc: Encoder, tap: int, dst) -> int:
    """Copy tap `tap` of the last encode into `dst`, a contiguous float32
    device tensor (its element count is the capacity the library checks)."""
    import torch
    if dst is None or not dst.is_cuda or dst.dtype != torch.float32 or not dst.is_contiguous():
        raise QAError(QA_STATUS_INVALID_PARAMS, "tap destination must be a contiguous float32 device tensor")
    n = _lib.qa_encoder_tap(enc.handle, tap, C.c_void_p(dst.data_ptr()), dst.numel())
    if n < 0:
        raise QAError(QA_STATUS_INVALID_PARAMS, qa_last_error())
    return n


def qa_encoder_set_profiling(enc: Encoder, enable: bool) -> None:
    _check(_lib.qa_encoder_set_profiling(enc.handle, 1 if enable else 0))


def qa_encoder_set_max_lanes(enc: Encoder, n: int) -> None:
    """The most streams an encode may run on: 1 (the handle's alone) to 4 (the default)."""
    _check(_lib.qa_encoder_set_max_lanes(enc.handle, int(n)))


def qa_encoder_set_profiling_label(enc: Encoder, label: Optional[str]) -> None:
    """Time only the launches labelled `label` (None: every launch)."""
    _check(_lib.qa_encoder_set_profiling_label(enc.handle, label.encode() if label else None))


def qa_encoder_kernel_times(enc: Encoder) -> Dict[str, tuple]:
    """label -> (total_ms, launches) since profiling was enabled."""
    n = _lib.qa_encoder_kernel_times(enc.handle, None, None, None, 0)
    labels = (C.c_char_p * max(n, 1))()
    ms = (C.c_double * max(n, 1))()
    cnt = (C.c_int64 * max(n, 1))()
    n = _lib.qa_encoder_kernel_times(enc.handle, labels, ms, cnt, n)
    return {labels[i].decode(): (ms[i], cnt[i]) for i in range(n)}


def qa_encoder_free(enc: Encoder) -> None:
    enc.free()


def encode(enc: Encoder, pcm, lengths: Sequence[int], out=None):
    """Allocate `out` (torch, on pcm's device) if needed and run qa_encode."""
    import torch
    counts = [qa_encode_num_tokens(int(x)) for x in lengths]
    for i, c in enumerate(counts):
        if c < 0:
            raise QAError(QA_STATUS_INVALID_PARAMS, f"clip {i}: {qa_last_error()}")
    total = sum(counts)
    if out is None:
        out = torch.empty((total, enc.dims.output_dim), dtype=torch.float32, device=pcm.device)
    qa_encode(enc, pcm, lengths, out)
    return out


# ------------------------------------------------------------------ resampler

class Resampler:
    """Owns a qa_resampler handle (the filter table for one input rate)."""

    def __init__(self, handle: int, rate: int):
        self.handle = handle
        self.rate = rate

    def __del__(self):
        self.free()

    def free(self):
        if getattr(self, "handle", None):
            _lib.qa_resampler_free(self.handle)
            self.handle = None


def qa_resample_length(n_in: int, rate_in: int) -> int:
    return _lib.qa_resample_length(int(n_in), int(rate_in))


def qa_resampler_create(rate_in: int) -> Resampler:
    h = _lib.qa_resampler_create(int(rate_in))
    if not h:
        raise QAError(QA_STATUS_INVALID_PARAMS, qa_last_error())
    return Resampler(h, int(rate_in))


def qa_resample(r: Resampler, stream, pcm_in, out) -> None:
    """pcm_in, out: contiguous float32 CUDA tensors; out must hold
    qa_resample_length(len(pcm_in), r.rate) samples."""
    import torch
    n = int(pcm_in.numel())
    need = qa_resample_length(n, r.rate)
    if pcm_in.dtype != torch.float32 or out.dtype != torch.float32 or not pcm_in.is_cuda or not out.is_cuda:
        raise QAError(QA_STATUS_INVALID_PARAMS, "pcm_in and out must be float32 device tensors")
    if not pcm_in.is_contiguous() or not out.is_contiguous() or out.numel() < need:
        raise QAError(QA_STATUS_INVALID_PARAMS, f"out must be contiguous with at least {need} samples")
    s = stream.cuda_stream if stream is not None and hasattr(stream, "cuda_stream") else (stream or 0)
    _check(_lib.qa_resample(r.handle, C.c_void_p(s), C.c_void_p(pcm_in.data_ptr()), n,
                            C.c_void_p(out.data_ptr())))


def resample(r: Resampler, pcm_in, stream=None):
    """Allocate the output on pcm_in's device and resample (asynchronous on `stream`,
    default: torch's current stream)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(pcm_in.device)
    out = torch.empty(max(qa_resample_length(int(pcm_in.numel()), r.rate), 0), dtype=torch.float32,
                      device=pcm_in.device)
    qa_resample(r, stream, pcm_in, out)
    return out



# ------------------------------------------------------------------ Thinker prefill

class Thinker:
    """Owns a qa_thinker handle."""

    def __init__(self, handle: int, dims: qa_thinker_dims):
        self.handle = handle
        self.dims = dims

    def __del__(self):
        self.free()

    def free(self):
        if getattr(self, "handle", None):
            _lib.qa_thinker_free(self.handle)
            self.handle = None


def make_thinker_dims(d) -> qa_thinker_dims:
    """qa_thinker_dims from any object/mapping with the ThinkerDims fields."""
    get = (lambda k: d[k]) if isinstance(d, Mapping) else (lambda k: getattr(d, k))
    dt = get("dtype")
    dt = {"f32": QA_DTYPE_F32, "bf16": QA_DTYPE_BF16}.get(dt, dt)
    return qa_thinker_dims(QA_ABI_VERSION, get("hidden"), get("n_layers"), get("n_q_heads"), get("n_kv_heads"),
                           get("head_dim"), get("ffn_dim"), get("vocab"), int(dt))


def qa_thinker_create(weights: Dict[str, np.ndarray], dims) -> Thinker:
    """weights: 'embed', 'out_norm' and 'layers.<l>.<field>' arrays in PyTorch layout."""
    qd = make_thinker_dims(dims)
    keep = []

    def ptr(name):
        b = _host_buffer(weights[name], qd.dtype)
        keep.append(b)
        return b.ctypes.data_as(C.c_void_p)

    w = qa_thinker_weights()
    w.embed = ptr("embed")
    w.out_norm = ptr("out_norm")
    L = qd.n_layers
    for n in THINKER_LAYER_FIELDS:
        arr = (C.c_void_p * max(L, 1))(*[ptr(f"layers.{l}.{n}") for l in range(L)])
        keep.append(arr)
        setattr(w, n, C.cast(arr, _VPP))
    h = _lib.qa_thinker_create(C.byref(w), C.byref(qd))
    if not h:
        raise QAError(QA_STATUS_LOAD_FAILED, qa_last_error())
    return Thinker(h, qd)


def qa_thinker_set_stream(t: Thinker, stream) -> None:
    raw = getattr(stream, "cuda_stream", stream)
    _check(_lib.qa_thinker_set_stream(t.handle, C.c_void_p(raw or 0)))


def qa_thinker_prefill(t: Thinker, prompts, audio, hidden_out=None, logits_out=None) -> None:
    """prompts: sequence of (ids int array, audio_offset, audio_count);
    audio: float32 CUDA tensor [sum counts, hidden] (or None when all counts
    are 0); hidden_out / logits_out: float32 CUDA tensors or None."""
    ids = np.ascontiguousarray(np.concatenate([np.asarray(p[0], dtype=np.int32) for p in prompts])
                               if prompts else np.zeros(0, np.int32))
    lens = np.ascontiguousarray([len(p[0]) for p in prompts], dtype=np.int64)
    offs = np.ascontiguousarray([int(p[1]) for p in prompts], dtype=np.int64)
    cnts = np.ascontiguousarray([int(p[2]) for p in prompts], dtype=np.int64)
    H, V = t.dims.hidden, t.dims.vocab
    A = int(cnts.sum()) if len(cnts) else 0

    import torch

    def dev(x, n, what):
        if x is None:
            return None
        if not x.is_cuda or x.dtype != torch.float32 or not x.is_contiguous() or x.numel() < n:
            raise QAError(QA_STATUS_INVALID_PARAMS, f"{what} must be a contiguous float32 device tensor of >= {n}")
        return C.c_void_p(x.data_ptr())

    pa = dev(audio, A * H, "audio") if A else None
    ph = dev(hidden_out, int(lens.sum()) * H, "hidden_out")
    pl = dev(logits_out, len(prompts) * V, "logits_out")
    _check(_lib.qa_thinker_prefill(t.handle, ids.ctypes.data_as(C.POINTER(C.c_int32)),
                                   lens.ctypes.data_as(C.POINTER(C.c_int64)), len(prompts), pa,
                                   offs.ctypes.data_as(C.POINTER(C.c_int64)),
                                   cnts.ctypes.data_as(C.POINTER(C.c_int64)), ph, pl))


def thinker_prefill(t: Thinker, prompts, audio, want_hidden: bool = True, want_logits: bool = True):
    """Allocate the outputs on audio's device (cuda:0 if audio is None) and prefill."""
    import torch
    devc = audio.device if audio is not None else torch.device("cuda:0")
    T = sum(len(p[0]) for p in prompts)
    h = torch.empty((T, t.dims.hidden), dtype=torch.float32, device=devc) if want_hidden else None
    g = torch.empty((len(prompts), t.dims.vocab), dtype=torch.float32, device=devc) if want_logits else None
    qa_thinker_prefill(t, prompts, audio, h, g)
    return h, g
