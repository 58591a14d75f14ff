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


def kernel_work(d, lengths):
    """Algorithmic work per launch of each labelled kernel: (flops, bytes,
    peak label).  Flops count dense MACs as 2; bytes count compulsory HBM
    traffic (operands read once, results written once)."""
    C, D, F, O, H = d.conv_channels, d.d_model, d.ffn_dim, d.output_dim, d.n_heads
    ch, T, fr, wins = plan_counts(lengths, window_chunks=d.window_chunks)
    e = 2 if d.dtype == "bf16" else 4
    work = {
        "frontend": (fr * (2 * 400 * 400 + 2 * 201 * 128), sum(lengths) * 4 + fr * 128 * 4, "fp32"),
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


# Source files whose kernels the HBM-traffic figure in profiles/ was taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "b17_20m_traffic.json")
KERNEL_SOURCES = ["audio_encoder_front_amd/csrc/" + f for f in
                  ("gemm.hip", "stem.hip", "frontend.hip", "norm_attn.hip", "encoder.cpp", "qa_device.h",
                   "qa_kernels.h")]


def sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
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
    if rec.get("workload") != workload or rec.get("kernel") != kernel or rec.get("sources") != sources_digest():
        return None
    return rec.get("bytes_per_launch")


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


def cpu_baseline(wl, seconds: float):
    """The fp64 oracle on the first `seconds` of the workload's first clip."""
    import numpy as np
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info()}))
    except Exception:  # pragma: no cover
        threads, blas = os.cpu_count(), "?"
    clip = synth.make_audio(wl)[0][: int(seconds * 16000)]
    w = synth.make_weights(wl.dims, wl.weight_seed)
    t0 = time.perf_counter()
    out = O.encode([clip], w, wl.dims.n_layers, wl.dims.n_heads, window_chunks=wl.dims.window_chunks)
    dt = time.perf_counter() - t0
    return {"value": len(clip) / 16000.0 / dt, "unit": "audio-s/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {seconds:g} s of the clip as one clip ({out.shape[0]} tokens), fp64 NumPy "
                      f"({blas}), {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="b17_20m")
    ap.add_argument("--cpu-sample-s", type=float, default=240.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-thinker", action="store_true", help="skip the Thinker-prefill line")
    ap.add_argument("--no-full-input", action="store_true", help="skip the full-input attention line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (reference for rocprofv3 byte counters)")
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
    dom = max((l for l in times if l in work), key=lambda l: times[l][0])
    # Timed steps: events only around the dominant kernel's launches.
    qa.qa_encoder_set_profiling_label(enc, dom)
    qa.qa_encoder_set_profiling(enc, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        qa.qa_encode(enc, pcm, lengths, out)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    dom_ms, dom_cnt = qa.qa_encoder_kernel_times(enc)[dom]
    qa.qa_encoder_set_profiling(enc, False)
    qa.qa_encoder_set_profiling_label(enc, None)

    audio_s = sum(lengths) / 16000.0
    ms_step = dt / args.steps * 1e3
    total_flops = sum(work[l][0] * cnt for l, (_, cnt) in times.items() if l in work) / prof_steps
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
        kernels[label] = ent
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
                   "tokens": T, "windows": len(wins), "chunks": n_chunks, "frames": n_frames},
        "tokens_per_s": round(T * args.steps / dt, 1),
        "mfma_util_pct": round(100.0 * total_flops / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 2),
        "roofline": roof,
        "kernels": kernels,
        "kernels_note": f"per-kernel table from {prof_steps} separate steps with events around every launch; "
                        "the timed steps carry events only around the dominant kernel",
    }
    res["resample"] = resample_bench(dev)
    if not args.no_full_input and wl.dims.window_chunks:
        res["full_input"] = full_input_bench(dev, wl, weights)
    del weights
    if not args.no_thinker:
        res["thinker_prefill"] = thinker_bench(dev, out, wl)
    if args.calibrate_copy:
        copy_calibration()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_s)
    enc.free()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
