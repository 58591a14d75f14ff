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


def compare(dims, weights, clips, gpu_out, gpu_taps, windows_per_clip=None, check_layer0=True):
    """Oracle on the same inputs; checks every (or the selected) window of
    every clip.  windows_per_clip: None (all) or a function (clip index,
    n_windows) -> list of window indices.  Returns a report dict."""
    W = O.as_f64(weights)
    tol_mel, tol_win, tol_stem = LOGMEL_TOL[dims.dtype], WINDOW_TOL[dims.dtype], STEM_TOL[dims.dtype]
    tok_off = 0
    frame_off = 0
    worst = {"log_mel": 0.0, "window": 0.0, "stem": 0.0, "layer0": 0.0, "windows_checked": 0}
    for ci, x in enumerate(clips):
        n = len(x)
        nt = O.clip_num_tokens(n)
        nf = n // 160
        if n == 0:
            continue
        win_tok = 13 * dims.window_chunks if dims.window_chunks else nt   # 0: one segment per clip
        nw = len(O.window_bounds(nt, win_tok))
        sel = None if windows_per_clip is None else sorted(set(windows_per_clip(ci, nw)))
        taps = {}
        ref = O.encode_clip(np.asarray(x, dtype=np.float64), W, dims.n_layers, dims.n_heads,
                            window_chunks=dims.window_chunks, windows=sel, taps=taps)
        if gpu_taps:
            g = gpu_taps["log_mel"][frame_off:frame_off + nf].T
            err = float(np.abs(g - taps["log_mel"]).max())
            assert err <= tol_mel, f"clip {ci}: log-mel max-abs {err:.3g} > {tol_mel}"
            worst["log_mel"] = max(worst["log_mel"], err)
        for wi, yref in ref.items():
            s = tok_off + wi * win_tok
            yg = gpu_out[s:s + yref.shape[0]]
            e = rel_l2(yg, yref)
            assert e <= tol_win, f"clip {ci} window {wi}: rel L2 {e:.3g} > {tol_win}"
            worst["window"] = max(worst["window"], e)
            worst["windows_checked"] += 1
            if gpu_taps:
                es = rel_l2(gpu_taps["stem"][s:s + yref.shape[0]], taps["stem"][wi])
                assert es <= tol_stem, f"clip {ci} window {wi}: stem rel L2 {es:.3g} > {tol_stem}"
                worst["stem"] = max(worst["stem"], es)
                if check_layer0 and dims.n_layers > 0:
                    el = rel_l2(gpu_taps["layer0"][s:s + yref.shape[0]], taps["layer0"][wi])
                    assert el <= tol_win, f"clip {ci} window {wi}: layer-0 rel L2 {el:.3g}"
                    worst["layer0"] = max(worst["layer0"], el)
        tok_off += nt
        frame_off += nf
    assert tok_off == gpu_out.shape[0]
    return worst


def workload_inputs(name):
    wl = synth.WORKLOADS[name]
    return wl, synth.make_audio(wl), synth.make_weights(wl.dims, wl.weight_seed)
