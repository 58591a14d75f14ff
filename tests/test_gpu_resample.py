"""GPU parity of the 16 kHz resampler (reading R1 of [qwenasr] "Module map")
against the oracle, through the C ABI.

Tolerance: each output is an fp32 FMA chain of at most L = ceil((2 half + 1) /
up) terms (21 at 8 kHz, 55 at 44.1 kHz, 961 at 768 kHz) with fp32-rounded
coefficients, so its error is below (L + 1) 2^-24 sum_j |h_j| |x_j| <=
(L + 1) 2^-24 max_p sum_j |h_pj| max|x|; the test uses that bound."""
import numpy as np
import pytest

import oracle.resample as R

pytestmark = pytest.mark.gpu

RATES = [44100, 48000, 22050, 8000, 11025, 96000, 44056, 16000, 1000, 768000]


def _signal(n, rate, seed):
    rng = np.random.default_rng(seed)
    t = np.arange(n) / rate
    x = 0.05 * rng.standard_normal(n)
    for f in rng.uniform(50, min(7000, 0.45 * rate), 3):
        x += 0.2 * np.sin(2 * np.pi * f * t + rng.uniform(0, 2 * np.pi))
    return x.astype(np.float32)


def _tol(rate, x):
    up, down, half, h = R.design(rate)
    L = -(-h.shape[0] // up)
    phase_sum = max(np.abs(h[p::up]).sum() for p in range(up))
    return (L + 1) * 2.0 ** -24 * phase_sum * max(float(np.abs(x).max()), 1e-30)


def _gpu(rate, x):
    import torch
    import audio_encoder_front_amd as qa
    r = qa.qa_resampler_create(rate)
    y = qa.resample(r, torch.from_numpy(x).to("cuda:0"))
    torch.cuda.synchronize()
    r.free()
    return y.cpu().double().numpy()


@pytest.mark.parametrize("rate", RATES)
def test_resample_matches_oracle(rate):
    for i, n in enumerate((1, 7, 1000, 12345)):
        x = _signal(n, rate, [rate, i])
        print("case: resample", rate, n, flush=True)
        y = _gpu(rate, x)
        ref = R.resample(x.astype(np.float64), rate)
        assert y.shape == ref.shape
        err = np.abs(y - ref).max()
        assert err <= _tol(rate, x), (rate, n, err, _tol(rate, x))


def test_resample_empty_and_rejections():
    import torch
    import audio_encoder_front_amd as qa
    r = qa.qa_resampler_create(44100)
    y = qa.resample(r, torch.zeros(0, device="cuda:0"))
    assert y.numel() == 0
    out = torch.empty(10, device="cuda:0")
    with pytest.raises(qa.QAError):       # output too small
        qa.qa_resample(r, None, torch.zeros(100, device="cuda:0"), out)
    r.free()
    with pytest.raises(qa.QAError):
        qa.qa_resampler_create(999)


def test_resample_twenty_minutes_44k1_sampled():
    # the full-size case: a 20-minute 44.1 kHz clip (52.92 M samples, the
    # longest request) -> 19.2 M samples, checked at the edges and at 3000
    # random outputs
    rate = 44100
    n = 20 * 60 * rate
    x = _signal(n, rate, 77)
    print("case: resample 20 min at 44.1 kHz", flush=True)
    y = _gpu(rate, x)
    assert y.shape == (19_200_000,)
    rng = np.random.default_rng(78)
    idx = np.concatenate([np.arange(50), np.arange(y.shape[0] - 50, y.shape[0]), rng.integers(0, y.shape[0], 3000)])
    ref = R.resample(x, rate, outputs=idx)
    err = np.abs(y[idx] - ref).max()
    assert err <= _tol(rate, x), (err, _tol(rate, x))
