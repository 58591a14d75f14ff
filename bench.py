"""Throughput of the AuT audio-encoder forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload b17_20m]

A step is one qa_encode of the whole batch: log-mel front end, conv stem,
every encoder layer and the output projection, with the PCM and the weights
already resident in HBM.  Prints one JSON line.  Per-kernel durations come
from HIP events the library records on its stream around every launch during
the timed steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "audio-sec encoded/sec (log-mel+AuT encoder), 1 MI355X; MFMA util %"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def log(msg: str) -> None:
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def plan_counts(lengths, chunk_tok=13, window_chunks=8):
    """Integer bookkeeping of the batch: chunks (tails padded to 100 frames
    count as full chunks of stem work), tokens, window sizes, frames."""
    chunks, tokens, frames, windows = 0, 0, 0, []
    for n in lengths:
        nf = n // 160
        frames += nf
        full, tail = divmod(nf, 100)
        chunks += full + (1 if tail else 0)
        t = full * chunk_tok + ((tail + 7) // 8 if tail else 0)
        tokens += t
        w = chunk_tok * window_chunks if window_chunks else max(t, 1)   # 0: one segment per clip
        windows += [min(w, t - s) for s in range(0, t, w)]
    return chunks, tokens, frames, windows


# The front end's DFT per STFT frame: 400 windowed samples against 201 cos and
# 201 sin basis rows, 2 * 400 * 402 = 321,600 flops of fp32 work (the sparse
# Slaney mel adds 2 * 394, on the VALU).  The kernel runs it on the bf16 MFMA
# as six products of exact three-part bf16 splits, on the MFMA-padded shape
# of 416 samples (13 K blocks of 32) x 208 bins (13 tiles of 16) x cos, sin:
# 6 * 2 * 416 * 208 * 2 = 2,076,672 bf16 MFMA flops per frame, the figure
# its roofline is stated against (the bf16 dense peak).
FRONT_FP32_FLOPS = 2 * 400 * 402
FRONT_BF16_EXEC_FLOPS = 6 * 2 * 416 * 208 * 2


def kernel_work(d, lengths):
    """Algorithmic work per launch of each labelled kernel: (flops, bytes,
    peak label).  Flops count dense MACs as 2; bytes count compulsory HBM
    traffic (operands read once, results written once).  The front end's
    flops are the bf16 MFMA flops it executes (FRONT_BF16_EXEC_FLOPS per
    frame, the final STFT frame of each clip included)."""
    C, D, F, O, H = d.conv_channels, d.d_model, d.ffn_dim, d.output_dim, d.n_heads
    ch, T, fr, wins = plan_counts(lengths, window_chunks=d.window_chunks)
    e = 2 if d.dtype == "bf16" else 4
    fr_all = fr + sum(1 for n in lengths if n)
    work = {
        "frontend": (fr_all * FRONT_BF16_EXEC_FLOPS, sum(lengths) * 4 + fr * 128 * 4, "bf16"),
        # conv1 + conv2 in one kernel (bf16 stems up to 512 channels): the
        # method's conv1 and conv2 flops; log-mel in, conv2's output and weights
        "stem12": (2 * ch * 64 * 50 * C * 9 + 2 * ch * 800 * C * 9 * C,
                   fr * 128 * 4 + ch * 800 * C * e + 9 * C * C * e, "bf16"),
        "conv2": (2 * ch * 800 * C * 9 * C, ch * 64 * 50 * C * e + ch * 800 * C * e + 9 * C * C * e, "bf16"),
        "conv3": (2 * ch * 208 * C * 9 * C, ch * 800 * C * e + ch * 208 * C * e + 9 * C * C * e, "bf16"),
        "conv_out": (2 * T * 16 * C * D, T * 16 * C * e + 16 * C * D * e + T * D * 4, "bf16"),
        "qkv": (2 * T * D * 3 * D, T * D * e + 3 * D * D * e + T * 3 * D * e, "bf16"),
        "attention": (sum(4 * n * n * 64 * H for n in wins), T * 3 * D * e + T * D * e, "bf16"),
        "o_proj": (2 * T * D * D, T * D * e + D * D * e + 2 * T * D * 4, "bf16"),
        "fc1": (2 * T * D * F, T * D * e + F * D * e + T * F * e, "bf16"),
        "fc2": (2 * T * F * D, T * F * e + F * D * e + 2 * T * D * 4, "bf16"),
        "proj1": (2 * T * D * D, T * D * e + D * D * e + T * D * e, "bf16"),
        "proj2": (2 * T * D * O, T * D * e + O * D * e + T * O * 4, "bf16"),
        "ln": (0, T * D * 4 + T * D * e, "hbm"),
        "conv1": (2 * ch * 64 * 50 * C * 9, fr * 128 * 4 + ch * 64 * 50 * C * e, "hbm"),
        "normalize": (0, 2 * fr * 128 * 4, "hbm"),
    }
    return work, (ch, T, fr, wins)


# Source files whose kernels the HBM-traffic figure in profiles/ was taken on:
# the kernel's own file and the headers it includes (every source for a
# kernel not listed).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "b17_20m_traffic.json")
KERNEL_SOURCES = ["audio_encoder_front_amd/csrc/" + f for f in
                  ("gemm.hip", "stem.hip", "stem_fused.hip", "frontend.hip", "norm_attn.hip", "encoder.cpp", "qa_device.h",
                   "qa_kernels.h")]
KERNEL_OWN_SOURCES = {
    "stem12": ["audio_encoder_front_amd/csrc/" + f for f in ("stem_fused.hip", "qa_device.h", "qa_kernels.h")],
    "fc1": ["audio_encoder_front_amd/csrc/" + f for f in ("gemm.hip", "qa_device.h", "qa_kernels.h")],
}


def sources_digest(kernel: str = None) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_OWN_SOURCES.get(kernel, KERNEL_SOURCES):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE measurement, or None if there is none for this
    kernel and workload or the kernel sources changed since it was taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if rec.get("workload") != workload or not k or k.get("sources") != sources_digest(kernel):
        return None
    return k.get("bytes_per_launch")


def copy_calibration(nbytes: int = 1 << 30):
    """One plain device-to-device copy of nbytes, the reference the HBM
    traffic counters are scaled against."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()


def resample_bench(dev, rate: int = 44100, seconds: int = 1200, reps: int = 10):
    """The resampler in front of the front end, timed on its own: one
    20-minute clip at 44.1 kHz to 16 kHz (not part of `value`)."""
    import numpy as np
    import torch
    import audio_encoder_front_amd as qa
    n = seconds * rate
    rng = np.random.default_rng(5)
    x = torch.from_numpy((0.1 * rng.standard_normal(n)).astype(np.float32)).to(dev)
    r = qa.qa_resampler_create(rate)
    out = torch.empty(qa.qa_resample_length(n, rate), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(2):
        qa.qa_resample(r, stream, x, out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        qa.qa_resample(r, stream, x, out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    r.free()
    nbytes = 4 * (n + out.numel())
    return {"workload": f"one {seconds} s clip at {rate} Hz -> 16 kHz", "avg_ms": round(ms, 4),
            "audio_s_per_s": round(seconds / (ms * 1e-3), 1), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "bound": "hbm", "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)}


def thinker_bench(dev, enc_out, wl, reps: int = 3):
    """The step after the encoder, timed on its own (not part of `value`): the
    Thinker of the same model size prefilling one prompt whose placeholder
    span is the encoder output just computed (all clips' states in one span)."""
    import numpy as np
    import torch
    import audio_encoder_front_amd as qa
    import synth.thinker as ST
    dims = ST.THINKER_17B if wl.dims.output_dim == ST.THINKER_17B.hidden else ST.THINKER_06B
    if enc_out.shape[1] != dims.hidden:
        return None
    W = ST.make_weights(dims, 317)
    t = qa.qa_thinker_create(W, dims)
    del W
    stream = torch.cuda.current_stream(dev)
    qa.qa_thinker_set_stream(t, stream)
    S = enc_out.shape[0]
    ids, off = ST.make_prompt(S, dims.vocab, [318, 0])
    prompts = [(ids, off, S)]
    T = len(ids)
    h = torch.empty((T, dims.hidden), dtype=torch.float32, device=dev)
    g = torch.empty((1, dims.vocab), dtype=torch.float32, device=dev)
    qa.qa_thinker_prefill(t, prompts, enc_out, h, g)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        qa.qa_thinker_prefill(t, prompts, enc_out, h, g)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / reps * 1e3
    t.free()
    H, F, hq, hkv, L = dims.hidden, dims.ffn_dim, dims.n_q_heads, dims.n_kv_heads, dims.n_layers
    gemm = 2.0 * T * (H * (hq + 2 * hkv) * 128 + hq * 128 * H + 2 * H * F + F * H) * L
    attn = 4.0 * (T * (T + 1) / 2) * 128 * hq * L          # QK^T and PV over the causal triangle
    flops = gemm + attn + 2.0 * H * dims.vocab
    return {"workload": f"{H}-hidden Thinker ({L} layers, {hq}/{hkv} heads of 128, FFN {F}) prefill of one "
                        f"prompt splicing the {S} encoder states ({T} tokens)",
            "avg_ms": round(ms, 3), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1), "flops": flops,
            "mfma_frac": round(flops / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4)}


def full_input_bench(dev, wl, weights, n_clips: int = 40, seconds: int = 30, steps: int = 5):
    """Full-input attention (one attention segment per clip, the variant for
    bounded inputs of at most 30 s), timed on its own (not part of `value`):
    the same encoder and weights with window_chunks = 0 on n_clips clips of
    `seconds` each (the same audio duration as the 20-minute workload)."""
    import dataclasses
    import numpy as np
    import torch
    import audio_encoder_front_amd as qa
    import synth
    dims = dataclasses.replace(wl.dims, window_chunks=0)
    enc = qa.qa_encoder_create(weights, dims)
    stream = torch.cuda.current_stream(dev)
    qa.qa_encoder_set_stream(enc, stream)
    clips = [synth.speech_like_clip(seconds * 16000, [wl.audio_seed + 1000, i]) for i in range(n_clips)]
    lengths = [len(c) for c in clips]
    pcm = torch.from_numpy(np.concatenate(clips)).to(dev)
    T = sum(qa.qa_encode_num_tokens(n) for n in lengths)
    out = torch.empty((T, dims.output_dim), dtype=torch.float32, device=dev)
    qa.qa_encode(enc, pcm, lengths, out)
    qa.qa_encoder_set_profiling(enc, True)
    qa.qa_encode(enc, pcm, lengths, out)
    torch.cuda.synchronize()
    times = qa.qa_encoder_kernel_times(enc)
    qa.qa_encoder_set_profiling(enc, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        qa.qa_encode(enc, pcm, lengths, out)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    enc.free()
    work, (_, _, _, segs) = kernel_work(dims, lengths)
    att_ms, att_n = times["attention"]
    att_avg = att_ms / max(att_n, 1)
    f, b, _ = work["attention"]
    return {"workload": f"{n_clips} clips x {seconds} s, one attention segment per clip "
                        f"({max(segs)} tokens), same encoder and weights",
            "audio_s_per_s": round(n_clips * seconds / dt, 1), "ms_per_step": round(dt * 1e3, 3),
            "attention": {"avg_ms": round(att_avg, 5), "launches": int(att_n),
                          "tflops": round(f / (att_avg * 1e-3) / 1e12, 1),
                          "frac_of_bf16_peak": round(f / (att_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "gbs": round(b / (att_avg * 1e-3) / 1e9, 1)}}


def cpu_baseline(wl, clips, weights, seconds: float = 0.0):
    """The fp64 oracle (as it stands) on the workload's clips, on the host's
    cores: per clip, its log-mel once, then oracle.encode_clip over groups of
    windows on one thread per usable core (one BLAS thread each; NumPy
    releases the GIL in its matmuls).  seconds > 0 takes only the first
    `seconds` of the first clip."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_info, threadpool_limits
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info()}))
    if seconds > 0:
        clips = [clips[0][: int(seconds * 16000)]]
    W = O.as_f64(weights)
    d = wl.dims
    t0 = time.perf_counter()
    tokens = 0
    with threadpool_limits(1), ThreadPoolExecutor(cores) as ex:
        for clip in clips:
            x = np.asarray(clip, dtype=np.float64)
            nt = O.clip_num_tokens(len(x))
            if nt == 0:
                continue
            mel = O.log_mel(x)
            wins = list(range(len(O.window_bounds(nt, 13 * d.window_chunks))))
            groups = [g for g in (wins[i::cores] for i in range(cores)) if g]
            outs = list(ex.map(lambda g: O.encode_clip(x, W, d.n_layers, d.n_heads, window_chunks=d.window_chunks,
                                                       windows=g, mel=mel), groups))
            tokens += sum(v.shape[0] for o in outs for v in o.values())
    dt = time.perf_counter() - t0
    audio = sum(len(c) for c in clips) / 16000.0
    what = f"first {seconds:g} s of the first clip" if seconds > 0 else f"the whole workload ({len(clips)} clip(s))"
    return {"value": audio / dt, "unit": "audio-s/s", "cores": cores, "kind": "oracle",
            "sample": f"{what}: {audio:g} s of audio, {tokens} tokens; fp64 NumPy ({blas}), the windows of a "
                      f"clip split over {cores} threads with one BLAS thread each; {dt:.1f} s wall"}


def vendor_block(dev, d, tokens: int, chunks: int, reps: int = 10):
    """The same contractions through the vendor libraries via torch (context,
    not part of `value`): the four encoder-layer GEMMs as torch.nn.functional
    .linear in bf16 (hipBLASLt; bias only, no fused GELU or residual) and conv2
    as conv2d in bf16 channels-last (MIOpen; bias only, no GELU), on random
    operands of the workload's shapes; median of `reps` timed calls."""
    import torch
    import torch.nn.functional as Fn
    g = torch.Generator(device=dev).manual_seed(7)
    D, F, C = d.d_model, d.ffn_dim, d.conv_channels
    s = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def med(fn):
        fn()
        t = []
        for _ in range(reps):
            e0.record(s)
            fn()
            e1.record(s)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1))
        return sorted(t)[len(t) // 2]

    def rnd(*shape):
        return (torch.randn(*shape, device=dev, generator=g) * 0.02).to(torch.bfloat16)

    res = {}
    for name, (k, n) in {"qkv": (D, 3 * D), "o_proj": (D, D), "fc1": (D, F), "fc2": (F, D)}.items():
        x, w, b = rnd(tokens, k), rnd(n, k), rnd(n)
        ms = med(lambda: Fn.linear(x, w, b))
        res[name] = {"avg_ms": round(ms, 4), "tflops": round(2.0 * tokens * k * n / (ms * 1e-3) / 1e12, 1)}
        del x, w, b
    x = rnd(chunks, C, 64, 50).contiguous(memory_format=torch.channels_last)
    w = rnd(C, C, 3, 3).contiguous(memory_format=torch.channels_last)
    b = rnd(C)
    ms = med(lambda: Fn.conv2d(x, w, b, stride=2, padding=1))
    res["conv2"] = {"avg_ms": round(ms, 4), "tflops": round(2.0 * chunks * 800 * C * 9 * C / (ms * 1e-3) / 1e12, 1)}
    del x, w, b
    torch.cuda.empty_cache()
    res["note"] = ("torch bf16 linear (hipBLASLt) and channels-last conv2d (MIOpen), bias only; "
                   "the encoder's own kernels also fuse GELU, the fp32 residual and the bf16 conversion")
    return res


def workload_block(dev, name, weights=None, steps: int = 10, warmup: int = 3):
    """Throughput of another benchmark workload through the same qa_encode
    (not part of `value`), with the roofline fraction of its dominant kernel
    from one step with events around every launch."""
    import numpy as np
    import torch
    import audio_encoder_front_amd as qa
    import synth
    wl = synth.WORKLOADS[name]
    clips = synth.make_audio(wl)
    lengths = [len(c) for c in clips]
    if weights is None:
        weights = synth.make_weights(wl.dims, wl.weight_seed)
    enc = qa.qa_encoder_create(weights, wl.dims)
    stream = torch.cuda.current_stream(dev)
    qa.qa_encoder_set_stream(enc, stream)
    pcm = torch.from_numpy(np.concatenate(clips)).to(dev)
    T = sum(qa.qa_encode_num_tokens(n) for n in lengths)
    out = torch.empty((T, wl.dims.output_dim), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        qa.qa_encode(enc, pcm, lengths, out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        qa.qa_encode(enc, pcm, lengths, out)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    qa.qa_encoder_set_profiling(enc, True)
    qa.qa_encode(enc, pcm, lengths, out)
    torch.cuda.synchronize()
    times = qa.qa_encoder_kernel_times(enc)
    qa.qa_encoder_set_profiling(enc, False)
    enc.free()
    work, (ch, _, fr, wins) = kernel_work(wl.dims, lengths)
    dom = max((l for l in times if l in work), key=lambda l: times[l][0])
    f, b, kind = work[dom]
    ms, cnt = times[dom]
    avg_s = ms / max(cnt, 1) * 1e-3
    total_flops = sum(work[l][0] * c for l, (_, c) in times.items() if l in work and l != "frontend")
    audio = sum(lengths) / 16000.0
    blk = {"workload": f"{name}: {wl.description}", "audio_s": round(audio, 2), "tokens": T, "windows": len(wins),
           "audio_s_per_s": round(audio / dt, 1), "tokens_per_s": round(T / dt, 1), "ms_per_step": round(dt * 1e3, 4),
           "mfma_util_pct": round(100.0 * total_flops / dt / (PEAK_BF16_TFLOPS * 1e12), 2),
           "dominant": {"kernel": dom, "avg_ms": round(avg_s * 1e3, 5), "launches": int(cnt),
                        "share_of_step": round(ms / (dt * 1e3), 3)}}
    if kind == "hbm":
        blk["dominant"].update(bound="hbm", gbs=round(b / avg_s / 1e9, 1), frac=round(b / avg_s / 1e9 / PEAK_HBM_GBS, 4))
    else:
        blk["dominant"].update(bound="mfma", tflops=round(f / avg_s / 1e12, 1),
                               frac=round(f / avg_s / 1e12 / PEAK_BF16_TFLOPS, 4))
    return blk


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="b17_20m")
    ap.add_argument("--cpu-sample-s", type=float, default=0.0,
                    help="oracle on the first N s of the first clip only (default 0: the whole workload)")
    ap.add_argument("--other-workloads", default="b06_1,b06_32,b17_16",
                    help="comma-separated workloads reported beside the main one ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-thinker", action="store_true", help="skip the Thinker-prefill line")
    ap.add_argument("--no-full-input", action="store_true", help="skip the full-input attention line")
    ap.add_argument("--vendor", action="store_true",
                    help="also time the layer GEMMs and conv2 through torch's vendor libraries (context)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (reference for rocprofv3 byte counters)")
    ap.add_argument("--lanes", type=int, default=4, choices=(1, 2, 3, 4),
                    help="the most streams the timed workload may run on (qa_encoder_set_max_lanes; the library "
                         "picks 2 or 3 lanes by batch size; 1 for per-kernel profiles whose dispatches all cover "
                         "the whole batch)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the encoder runs on a single MI355X and the library has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import audio_encoder_front_amd as qa
    import synth

    wl = synth.WORKLOADS[args.workload]
    clips = synth.make_audio(wl)
    lengths = [len(c) for c in clips]
    weights = synth.make_weights(wl.dims, wl.weight_seed)
    dev = torch.device("cuda:0")
    pcm = torch.from_numpy(np.concatenate(clips)).to(dev)
    enc = qa.qa_encoder_create(weights, wl.dims)
    stream = torch.cuda.current_stream(dev)
    qa.qa_encoder_set_stream(enc, stream)
    qa.qa_encoder_set_max_lanes(enc, args.lanes)
    total_tok = sum(qa.qa_encode_num_tokens(n) for n in lengths)
    out = torch.empty((total_tok, wl.dims.output_dim), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        qa.qa_encode(enc, pcm, lengths, out)
    torch.cuda.synchronize()
    # Per-kernel table: separate, untimed steps with events around every launch.
    prof_steps = 2
    qa.qa_encoder_set_profiling(enc, True)
    for _ in range(prof_steps):
        qa.qa_encode(enc, pcm, lengths, out)
    torch.cuda.synchronize()
    times = qa.qa_encoder_kernel_times(enc)
    qa.qa_encoder_set_profiling(enc, False)
    work, (n_chunks, T, n_frames, wins) = kernel_work(wl.dims, lengths)
    # dominant kernel: largest total time among the labelled compute kernels
    # (these steps run as one lane: every launch covers the whole batch)
    dom = max((l for l in times if l in work), key=lambda l: times[l][0])
    # Timed steps: the value, no events.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        qa.qa_encode(enc, pcm, lengths, out)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    # Roofline steps: events around the dominant kernel's launches only, at one
    # lane, so that each timed launch does the whole batch's work (with lanes a
    # layer kernel runs as two or three launches over parts of the batch, side
    # by side with the other lanes' kernels); the kernel-trace profile of the
    # same kernel is taken at one lane as well.
    roof_steps = max(3, min(args.steps, 10))
    qa.qa_encoder_set_max_lanes(enc, 1)
    qa.qa_encoder_set_profiling_label(enc, dom)
    qa.qa_encoder_set_profiling(enc, True)
    torch.cuda.synchronize()
    for _ in range(roof_steps):
        qa.qa_encode(enc, pcm, lengths, out)
    torch.cuda.synchronize()
    dom_ms, dom_cnt = qa.qa_encoder_kernel_times(enc)[dom]
    qa.qa_encoder_set_profiling(enc, False)
    qa.qa_encoder_set_profiling_label(enc, None)
    qa.qa_encoder_set_max_lanes(enc, args.lanes)

    audio_s = sum(lengths) / 16000.0
    ms_step = dt / args.steps * 1e3
    # algorithmic flops of the step (the front end's bf16 split products are
    # not the method's work: it counts with its fp32 DFT flops)
    total_flops = sum(work[l][0] * cnt for l, (_, cnt) in times.items() if l in work and l != "frontend") / prof_steps
    total_flops += n_frames * FRONT_FP32_FLOPS
    kernels = {}
    for label, (ms, cnt) in sorted(times.items()):
        avg = ms / max(cnt, 1)
        ent = {"avg_ms": round(avg, 5), "launches": int(cnt), "total_ms_per_step": round(ms / prof_steps, 4)}
        if label in work:
            f, b, kind = work[label]
            if f:
                ent["tflops"] = round(f / (avg * 1e-3) / 1e12, 2)
            if b:
                ent["gbs"] = round(b / (avg * 1e-3) / 1e9, 1)
            if kind == "hbm":
                ent["frac_of_hbm_peak"] = round(b / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
            elif f:
                ent["frac_of_bf16_peak"] = round(f / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        kernels[label] = ent
    kernels["frontend"]["note"] = (f"tflops = executed bf16 MFMA flops ({FRONT_BF16_EXEC_FLOPS} per frame: six "
                                   f"split products on the padded 416 x 208 x 2 DFT) against the bf16 peak; the "
                                   f"DFT's fp32 work is {FRONT_FP32_FLOPS} flops per frame")
    f, b, kind = work[dom]
    avg_s = dom_ms / max(dom_cnt, 1) * 1e-3
    if kind == "hbm":
        roof = {"bound": "hbm", "achieved": b / avg_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        peak = PEAK_BF16_TFLOPS if kind == "bf16" else PEAK_FP32_MFMA_TFLOPS
        roof = {"bound": "mfma", "achieved": f / avg_s / 1e12, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom, wl.name)
    roof["kernel"] = dom
    roof["per_launch"] = {"flops": f, "bytes": b}
    roof["avg_ms"] = round(avg_s * 1e3, 5)
    roof["launches_timed"] = int(dom_cnt)
    roof["timing"] = (f"HIP events around each launch of the kernel on its stream, {roof_steps} steps at one "
                      f"lane after the timed steps (every launch covers the whole batch)")
    res = {
        "metric": METRIC,
        "value": round(audio_s * args.steps / dt, 2),
        "unit": "audio-s/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dims.dtype,
        "data": "synthetic (seeded speech-like PCM, N(0,0.02) bf16 weights)",
        "config": {"workload": f"{wl.name}: {wl.description}", "clips": len(lengths), "audio_s": audio_s,
                   "tokens": T, "windows": len(wins), "chunks": n_chunks, "frames": n_frames,
                   "max_streams": args.lanes},
        "tokens_per_s": round(T * args.steps / dt, 1),
        "mfma_util_pct": round(100.0 * total_flops / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 2),
        "roofline": roof,
        # the whole step against the time its algorithmic flops need at the bf16 peak
        "step_roofline": {"algorithmic_tflop": round(total_flops / 1e12, 3),
                          "nameplate_ms": round(total_flops / PEAK_BF16_TFLOPS / 1e9, 3),
                          "frac_of_nameplate": round(total_flops / PEAK_BF16_TFLOPS / 1e9 / ms_step, 4)},
        "kernels": kernels,
        "kernels_note": f"per-kernel table from {prof_steps} separate steps at one lane with events around every "
                        "launch; the timed steps carry no events",
    }
    log(f"{wl.name}: {res['value']} audio-s/s, {ms_step:.3f} ms per step")
    # ceilings measured on this GPU in this run (register-only MFMA loop, HBM streaming)
    try:
        from audio_encoder_front_amd import probe
        res["ceilings"] = probe.measure(dev)
        c = res["ceilings"]
        meas = c["mfma_bf16_random_tflops"] if roof["unit"] == "TFLOP/s" else c["hbm_read_gbs"]
        roof["measured_ceiling"] = meas
        roof["frac_of_measured_ceiling"] = roof["achieved"] / meas
        res["step_roofline"]["measured_ceiling_ms"] = round(total_flops / (meas_mfma := c["mfma_bf16_random_tflops"]) / 1e9, 3)
        res["step_roofline"]["frac_of_measured"] = round(total_flops / meas_mfma / 1e9 / ms_step, 4)
        for ent in kernels.values():
            if "frac_of_bf16_peak" in ent:
                ent["frac_of_measured_mfma"] = round(ent["tflops"] / c["mfma_bf16_random_tflops"], 4)
            elif "frac_of_hbm_peak" in ent:
                ent["frac_of_measured_hbm"] = round(ent["gbs"] / c["hbm_read_gbs"], 4)
        res["ceilings"]["note"] = ("bf16 MFMA: register-only loop of 16x16x32 MFMAs with random full-mantissa "
                                   "operands (and all-ones operands); HBM: 1 GiB streaming read and copy; best of 5")
        log(f"ceilings: {c}")
    except (ImportError, OSError, RuntimeError) as ex:   # the probe library is optional for the encoder
        res["ceilings"] = {"error": str(ex)}
    res["resample"] = resample_bench(dev)
    log("resampler done")
    if not args.no_full_input and wl.dims.window_chunks:
        res["full_input"] = full_input_bench(dev, wl, weights)
        log("full-input attention done")
    others = [w for w in args.other_workloads.split(",") if w and w != wl.name]
    if others:
        res["other_workloads"] = {}
        for name in others:
            same = synth.WORKLOADS[name].dims == wl.dims and synth.WORKLOADS[name].weight_seed == wl.weight_seed
            res["other_workloads"][name] = workload_block(dev, name, weights if same else None)
            torch.cuda.empty_cache()
            log(f"{name}: {res['other_workloads'][name]['audio_s_per_s']} audio-s/s")
    if not args.no_thinker:
        res["thinker_prefill"] = thinker_bench(dev, out, wl)
        log("thinker prefill done")
    if args.vendor:
        res["vendor"] = vendor_block(dev, wl.dims, T, n_chunks)
        log(f"vendor libraries: {res['vendor']}")
    if args.calibrate_copy:
        copy_calibration()
    enc.free()
    if not args.no_cpu_baseline:
        log("cpu baseline (the oracle on the host) ...")
        res["cpu_baseline"] = cpu_baseline(wl, clips, weights, args.cpu_sample_s)
        log(f"cpu baseline: {res['cpu_baseline']['sample']}")
    del weights
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
