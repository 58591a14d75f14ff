"""Shared helpers of the GPU parity tests: run the HIP library through the
binding on seeded inputs and compare with the oracle window by window."""
from __future__ import annotations

import numpy as np

import oracle as O
import synth

LOGMEL_TOL = {"f32": 1e-4, "bf16": 2e-3}     # max-abs on the normalised log-mel
WINDOW_TOL = {"f32": 1e-4, "bf16": 1e-2}     # per-window relative L2 on the output
STEM_TOL = {"f32": 1e-4, "bf16": 1e-2}       # relative L2 of the pre-PE stem output per window


def device():
    import torch
    return torch.device("cuda:0")


def make_encoder(dims, weights):
    import audio_encoder_front_amd as qa
    return qa.qa_encoder_create(weights, dims)


def run_gpu(enc, clips, taps=False):
    """Returns (out [T, out_dim] float64 numpy, taps dict or None)."""
    import torch
    import audio_encoder_front_amd as qa
    lens = [int(len(c)) for c in clips]
    pcm = torch.from_numpy(np.concatenate(clips).astype(np.float32) if clips and sum(lens) else
                           np.zeros(0, np.float32)).to(device())
    qa.qa_encoder_enable_taps(enc, taps)
    qa.qa_encoder_set_stream(enc, torch.cuda.current_stream())
    out = qa.encode(enc, pcm, lens)
    torch.cuda.synchronize()
    res = {}
    if taps:
        n_frames = sum(l // 160 for l in lens)
        T = out.shape[0]
        d = enc.dims.d_model
        mel = torch.empty(n_frames * 128, dtype=torch.float32, device=device())
        qa.qa_encoder_tap(enc, qa._binding.QA_TAP_LOG_MEL, mel)
        stem = torch.empty(T * d, dtype=torch.float32, device=device())
        qa.qa_encoder_tap(enc, qa._binding.QA_TAP_STEM, stem)
        res["log_mel"] = mel.view(n_frames, 128).cpu().double().numpy()
        res["stem"] = stem.view(T, d).cpu().double().numpy()
        if enc.dims.n_layers > 0:
            l0 = torch.empty(T * d, dtype=torch.float32, device=device())
            qa.qa_encoder_tap(enc, qa._binding.QA_TAP_LAYER0, l0)
            res["layer0"] = l0.view(T, d).cpu().double().numpy()
    return out.cpu().double().numpy(), res


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def row_rel_l2(a, b):
    """Largest relative L2 error over the rows (tokens) of a block.  A row
    averages d (or out_dim) independent rounding errors, as many as a window's
    norm does per row, so its expected value is the window's and the window
    tolerance applies to it; it catches a defect confined to a few rows (one
    M tile, the tail rows of a chunk) that the window norm dilutes."""
    num = np.linalg.norm(a - b, axis=1)
    den = np.maximum(np.linalg.norm(b, axis=1), 1e-300)
    return float((num / den).max()) if a.shape[0] else 0.0


def _oracle_windows(x, W, dims, sel, threads):
    """encode_clip over the selected windows (all if None), split over a pool
    of threads (NumPy releases the GIL in its matmuls; BLAS runs one thread
    per call meanwhile).  Returns (outputs by window, taps)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    xd = np.asarray(x, dtype=np.float64)
    mel = O.log_mel(xd)
    nt = O.clip_num_tokens(len(x))
    win_tok = 13 * dims.window_chunks if dims.window_chunks else nt
    wins = list(range(len(O.window_bounds(nt, win_tok)))) if sel is None else list(sel)
    groups = [wins[i::threads] for i in range(threads)] if threads > 1 else [wins]
    groups = [g for g in groups if g]

    def run(g):
        taps = {}
        out = O.encode_clip(xd, W, dims.n_layers, dims.n_heads, window_chunks=dims.window_chunks,
                            windows=g, taps=taps, mel=mel)
        return out, taps

    if len(groups) <= 1:
        res = [run(g) for g in groups]
    else:
        with threadpool_limits(1), ThreadPoolExecutor(len(groups)) as ex:
            res = list(ex.map(run, groups))
    out, taps = {}, {"log_mel": mel, "stem": {}, "layer0": {}}
    for o, t in res:
        out.update(o)
        taps["stem"].update(t.get("stem", {}))
        taps["layer0"].update(t.get("layer0", {}))
    return out, taps


def oracle_threads():
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def compare(dims, weights, clips, gpu_out, gpu_taps, windows_per_clip=None, check_layer0=True, progress=None):
    """Oracle on the same inputs; checks every (or the selected) window of
    every clip, per window (relative L2) and per row (largest row relative
    L2), for the output and, with taps, the pre-PE stem and the layer-0
    residual.  windows_per_clip: None (all) or a function (clip index,
    n_windows) -> list of window indices.  progress: a label to print a line
    per clip with.  Returns a report dict."""
    W = O.as_f64(weights)
    tol_mel, tol_win, tol_stem = LOGMEL_TOL[dims.dtype], WINDOW_TOL[dims.dtype], STEM_TOL[dims.dtype]
    tok_off = 0
    frame_off = 0
    worst = {"log_mel": 0.0, "window": 0.0, "row": 0.0, "stem": 0.0, "stem_row": 0.0, "layer0": 0.0,
             "layer0_row": 0.0, "windows_checked": 0}
    threads = oracle_threads()
    for ci, x in enumerate(clips):
        n = len(x)
        nt = O.clip_num_tokens(n)
        nf = n // 160
        if n == 0:
            continue
        win_tok = 13 * dims.window_chunks if dims.window_chunks else nt   # 0: one segment per clip
        nw = len(O.window_bounds(nt, win_tok))
        sel = None if windows_per_clip is None else sorted(set(windows_per_clip(ci, nw)))
        ref, taps = _oracle_windows(x, W, dims, sel, threads)
        if gpu_taps:
            g = gpu_taps["log_mel"][frame_off:frame_off + nf].T
            err = float(np.abs(g - taps["log_mel"]).max())
            assert err <= tol_mel, f"clip {ci}: log-mel max-abs {err:.3g} > {tol_mel}"
            worst["log_mel"] = max(worst["log_mel"], err)
        for wi in sorted(ref):
            yref = ref[wi]
            s = tok_off + wi * win_tok
            yg = gpu_out[s:s + yref.shape[0]]
            e, er = rel_l2(yg, yref), row_rel_l2(yg, yref)
            assert e <= tol_win, f"clip {ci} window {wi}: rel L2 {e:.3g} > {tol_win}"
            assert er <= tol_win, f"clip {ci} window {wi}: a row's rel L2 {er:.3g} > {tol_win}"
            worst["window"] = max(worst["window"], e)
            worst["row"] = max(worst["row"], er)
            worst["windows_checked"] += 1
            if gpu_taps:
                gs, rs = gpu_taps["stem"][s:s + yref.shape[0]], taps["stem"][wi]
                es, esr = rel_l2(gs, rs), row_rel_l2(gs, rs)
                assert es <= tol_stem, f"clip {ci} window {wi}: stem rel L2 {es:.3g} > {tol_stem}"
                assert esr <= tol_stem, f"clip {ci} window {wi}: a stem row's rel L2 {esr:.3g} > {tol_stem}"
                worst["stem"] = max(worst["stem"], es)
                worst["stem_row"] = max(worst["stem_row"], esr)
                if check_layer0 and dims.n_layers > 0:
                    gl, rl = gpu_taps["layer0"][s:s + yref.shape[0]], taps["layer0"][wi]
                    el, elr = rel_l2(gl, rl), row_rel_l2(gl, rl)
                    assert el <= tol_win, f"clip {ci} window {wi}: layer-0 rel L2 {el:.3g}"
                    assert elr <= tol_win, f"clip {ci} window {wi}: a layer-0 row's rel L2 {elr:.3g}"
                    worst["layer0"] = max(worst["layer0"], el)
                    worst["layer0_row"] = max(worst["layer0_row"], elr)
        if progress:
            print(f"{progress}: clip {ci + 1}/{len(clips)}, {len(ref)} windows checked, worst so far "
                  f"window {worst['window']:.3g} row {worst['row']:.3g}", flush=True)
        tok_off += nt
        frame_off += nf
    assert tok_off == gpu_out.shape[0]
    return worst


def tail_reading_check(dims, weights, clips, gpu_taps, margin=10.0):
    """The tail-chunk reading (A: the chunk's log-mel zero-padded to 100
    frames, the whole stem run, the first f3(m) rows kept; B: the stem run on
    the m frames): for every clip whose tail chunk's last row differs between
    the two readings by more than `margin` times the stem tolerance, that GPU
    row must match reading A within the tolerance (and so not B).  Returns
    the rows checked as (clip, m, error vs A, error vs B)."""
    W = O.as_f64(weights)
    tol = STEM_TOL[dims.dtype]
    tok_off = 0
    checked = []
    for ci, x in enumerate(clips):
        n = len(x)
        nt = O.clip_num_tokens(n)
        if n == 0:
            continue
        lens = O.chunk_lengths(n // 160)
        m = lens[-1]
        if m < 100:
            mel = O.log_mel(np.asarray(x, dtype=np.float64))
            chunk = mel[:, mel.shape[1] - m:]
            a = O.stem_chunk(chunk, W, m, "A")[-1]
            b = O.stem_chunk(chunk, W, m, "B")[-1]
            g = gpu_taps["stem"][tok_off + nt - 1]
            ea, eb, ab = rel_l2(g, a), rel_l2(g, b), rel_l2(b, a)
            if ab > margin * tol:
                assert ea <= tol, f"clip {ci} (tail {m} frames): last row vs reading A {ea:.3g} > {tol}"
                assert eb > (margin - 1) * tol, f"clip {ci}: last row is as close to reading B ({eb:.3g})"
                checked.append((ci, m, ea, eb))
        tok_off += nt
    return checked


def workload_inputs(name):
    wl = synth.WORKLOADS[name]
    return wl, synth.make_audio(wl), synth.make_weights(wl.dims, wl.weight_seed)
