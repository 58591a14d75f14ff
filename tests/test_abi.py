"""C ABI checks that need no GPU: the library loads and exports every entry
point the public header declares, the token-count closed form agrees with the
oracle's planner, and every early-return path rejects bad arguments before
touching a device (including a strict-C99 consumer of the header)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as O
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qa_encoder.h")


@pytest.fixture(scope="module")
def qa():
    import audio_encoder_front_amd as qa
    return qa


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qa_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("qa_encoder_create", "qa_encode", "qa_encode_num_tokens", "qa_encoder_free", "qa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(qa):
    lib = qa.library()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(qa._binding.EXPORTS)
    # only qa_* symbols are exported
    out = subprocess.run(["nm", "-D", "--defined-only", qa._binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = [l.split()[-1] for l in out.splitlines() if l.split()[-2] in ("T", "W")]
    assert all(s.startswith("qa_") or s.startswith("_") for s in syms), syms


def test_num_tokens_matches_oracle_planner(qa):
    rng = np.random.default_rng(20)
    lens = [0, 201, 359, 16000, 16159, 16160, 32000, 480000, 19_200_000] + list(rng.integers(201, 19_200_000, 200))
    for n in lens:
        assert qa.qa_encode_num_tokens(int(n)) == O.clip_num_tokens(int(n)), n
    for wl in synth.WORKLOADS.values():
        for n in synth.clip_lengths(wl):
            assert qa.qa_encode_num_tokens(int(n)) == O.clip_num_tokens(int(n))


@pytest.mark.parametrize("n", [-1, 1, 100, 200, 19_200_001])
def test_num_tokens_rejects_invalid(qa, n):
    assert qa.qa_encode_num_tokens(n) == -1
    assert qa.qa_last_error()
    with pytest.raises(O.InvalidInput):
        O.validate_clip(n)


def _tiny_weights():
    return synth.make_weights(synth.DIMS_TINY, 100)


@pytest.mark.parametrize("field,value", [("n_mels", 80), ("head_dim", 32), ("chunk_frames", 50),
                                         ("window_chunks", -1), ("window_chunks", 10), ("conv_channels", 48),
                                         ("d_model", 200), ("n_heads", 3), ("ffn_dim", 1000),
                                         ("output_dim", 250), ("n_layers", -1), ("dtype", 5)])
def test_create_rejects_bad_dims(qa, field, value):
    d = qa.make_dims(synth.DIMS_TINY)
    setattr(d, field, value)
    w = qa._binding.qa_weights()
    assert qa.library().qa_encoder_create(ctypes.byref(w), ctypes.byref(d)) is None
    assert qa.qa_last_error()


def test_create_rejects_abi_mismatch_and_null_weights(qa):
    d = qa.make_dims(synth.DIMS_TINY)
    d.abi_version = 99
    w = qa._binding.qa_weights()
    assert qa.library().qa_encoder_create(ctypes.byref(w), ctypes.byref(d)) is None
    assert "abi_version" in qa.qa_last_error()
    d.abi_version = 1
    assert qa.library().qa_encoder_create(ctypes.byref(w), ctypes.byref(d)) is None
    assert "NULL" in qa.qa_last_error()


def test_bf16_weights_must_be_representable(qa):
    w = _tiny_weights()
    with pytest.raises(ValueError):
        qa._binding._host_buffer(np.float32([1.0 + 2 ** -12]), qa._binding.QA_DTYPE_BF16)
    assert qa._binding._host_buffer(w["conv1_w"], qa._binding.QA_DTYPE_F32).dtype == np.float32


def test_encode_rejects_bad_arguments_without_a_device(qa):
    lib = qa.library()
    lens = (ctypes.c_int64 * 2)(32000, 0)
    assert lib.qa_encode(None, None, lens, 2, None) == qa._binding.QA_STATUS_INVALID_PARAMS
    assert lib.qa_encoder_tap(None, 0, None, 0) == -1
    assert lib.qa_encoder_set_max_lanes(None, 1) == qa._binding.QA_STATUS_INVALID_PARAMS


def test_strict_c99_consumer(tmp_path, qa):
    exe = tmp_path / "abi_c"
    lib_dir = os.path.dirname(qa._binding.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "abi_c.c"), "-o", str(exe), "-L", lib_dir, "-lqa_encoder",
           "-Wl,-rpath," + lib_dir]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr + r.stdout


def test_resample_length_matches_oracle(qa):
    import oracle.resample as R
    rng = np.random.default_rng(21)
    for rate in (44100, 48000, 8000, 22050, 11025, 96000, 16000, 44056, 1000, 768000):
        for n in [0, 1, 2, 441, 44100] + list(rng.integers(1, 60_000_000, 20)):
            assert qa.qa_resample_length(int(n), rate) == R.output_length(int(n), rate), (rate, n)
    assert qa.qa_resample_length(-1, 44100) == -1
    assert qa.qa_resample_length(10, 999) == -1
    with pytest.raises(qa.QAError):
        qa.qa_resampler_create(768001)


def test_binding_checks_lengths_and_tap_buffers_before_the_library(qa):
    """encode() refuses an invalid clip length before it sizes `out`, and
    qa_encoder_tap refuses a destination that is not a contiguous float32
    device tensor (the library copies 4 bytes per counted element)."""
    import torch
    enc = qa._binding.Encoder(None, qa._binding.make_dims(synth.DIMS_TINY))
    with pytest.raises(qa.QAError) as ei:
        qa.encode(enc, torch.zeros(300), [300, 150])
    assert ei.value.status == qa._binding.QA_STATUS_INVALID_PARAMS and "clip 1" in str(ei.value)
    for dst in (torch.zeros(8), torch.zeros(8, dtype=torch.bfloat16)):
        with pytest.raises(qa.QAError):
            qa.qa_encoder_tap(enc, qa._binding.QA_TAP_LOG_MEL, dst)


def test_probe_library_exports_its_header():
    """libqa_probe.so (the benchmark's ceiling probes) exports what
    include/qa_probe.h declares."""
    from audio_encoder_front_amd import probe
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "qa_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(qa_[a-z_0-9]+)\s*\(", src)))
    assert len(names) == 4
    lib = probe._load()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.qa_probe_mfma_flops(2, 3) == 2 * 4 * 3 * 32 * 16 * 16 * 32 * 2
    assert lib.qa_probe_mfma_bf16(None, 0, 1, 1, None) == -1
    assert lib.qa_probe_read(None, None, 1024, None) == -1
