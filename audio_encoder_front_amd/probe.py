"""ctypes binding of libqa_probe.so: the ceiling probes the benchmark runs
beside the encoder (bf16 MFMA loop, HBM streaming).  Not the encoder's path."""
from __future__ import annotations

import ctypes as C
import os

PROBE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqa_probe.so")


def _load() -> C.CDLL:
    import torch  # noqa: F401  (bind to torch's HIP runtime, as the encoder library does)
    if not os.path.exists(PROBE_PATH):
        raise ImportError(f"{PROBE_PATH} is not built; run audio_encoder_front_amd.build.build()")
    lib = C.CDLL(PROBE_PATH)
    lib.qa_probe_mfma_bf16.restype = C.c_int
    lib.qa_probe_mfma_bf16.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p]
    lib.qa_probe_mfma_flops.restype = C.c_double
    lib.qa_probe_mfma_flops.argtypes = [C.c_int, C.c_int]
    lib.qa_probe_read.restype = C.c_int
    lib.qa_probe_read.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]
    lib.qa_probe_copy.restype = C.c_int
    lib.qa_probe_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64]
    return lib


def measure(dev, reps: int = 5):
    """Ceilings on this GPU now: bf16 MFMA TFLOP/s (random and constant
    operands) and HBM GB/s (1 GiB read, 1 GiB copy counted as read + write),
    each the best of `reps` timed launches after one warm-up."""
    import torch
    lib = _load()
    s = torch.cuda.current_stream(dev)
    sp = C.c_void_p(s.cuda_stream)
    scratch = torch.zeros(1, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn):
        fn()
        t = []
        for _ in range(reps):
            e0.record(s)
            fn()
            e1.record(s)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e-3)
        return min(t)

    res = {}
    blocks, iters = 1024, 5000
    fl = lib.qa_probe_mfma_flops(blocks, iters)
    for name, rnd in (("mfma_bf16_random_tflops", 1), ("mfma_bf16_const_tflops", 0)):
        sec = best(lambda: _ok(lib.qa_probe_mfma_bf16(sp, blocks, iters, rnd, C.c_void_p(scratch.data_ptr()))))
        res[name] = round(fl / sec / 1e12, 1)
    nbytes = 1 << 30
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    sec = best(lambda: _ok(lib.qa_probe_read(sp, C.c_void_p(a.data_ptr()), nbytes, C.c_void_p(scratch.data_ptr()))))
    res["hbm_read_gbs"] = round(nbytes / sec / 1e9, 1)
    sec = best(lambda: _ok(lib.qa_probe_copy(sp, C.c_void_p(a.data_ptr()), C.c_void_p(b.data_ptr()), nbytes)))
    res["hbm_copy_gbs"] = round(2 * nbytes / sec / 1e9, 1)
    del a, b
    return res


def _ok(status: int) -> None:
    if status != 0:
        raise RuntimeError(f"probe launch failed ({status})")
