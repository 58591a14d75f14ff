"""The GELU the kernels evaluate (qa_device.h: relu(z) - a exp2(P(a)),
a = min(|z|, A), Horner in fp32) against the exact erf GELU, with the
coefficients read from the kernel header itself: the error bounds the header
states hold over the fp32 range, and the fit in gelu_coeffs.py reproduces the
header's coefficients."""
import os
import re

import numpy as np
import scipy.special as sp

from audio_encoder_front_amd import gelu_coeffs as GC

HEADER = os.path.join(os.path.dirname(__file__), "..", "audio_encoder_front_amd", "csrc", "qa_device.h")
BOUND = {"gelu_erf": 2.7e-7, "gelu_erf_bf16": 6.4e-6}     # as stated in the header


def header_coeffs(name):
    src = open(HEADER).read()
    body = src[src.index(f"float {name}(float z)"):]
    body = body[:body.index("return")]
    clamp = float(re.search(r"fmed3f\(fabsf\(z\), 0\.0f, ([0-9.]+)f\)", body).group(1))
    vals = [float(v) for v in re.findall(r"([-+]?[0-9]\.[0-9]+e[-+][0-9]+)f", body)]
    return np.array(vals[::-1], dtype=np.float32), clamp       # lowest degree first


def test_header_gelu_within_stated_bounds():
    z = np.linspace(-40, 40, 2_000_001).astype(np.float32)
    zd = z.astype(np.float64)
    exact = 0.5 * zd * (1 + sp.erf(zd / np.sqrt(2.0)))
    for name, (deg, clamp) in GC.VARIANTS.items():
        coef, hclamp = header_coeffs(name)
        assert len(coef) == deg + 1 and hclamp == clamp, name
        err = np.abs(GC.gelu_f32(z, coef, clamp).astype(np.float64) - exact)
        assert err.max() <= BOUND[name], (name, err.max())
        # large |z|: exact relu on the positive side, a tiny negative tail
        big = np.array([60.0, -60.0, np.inf, -np.inf], np.float32)
        out = GC.gelu_f32(big, coef, clamp)
        assert out[0] == 60.0 and out[2] == np.inf and -2e-6 <= out[1] <= 0 and -2e-6 <= out[3] <= 0


def test_fit_reproduces_header_coefficients():
    for name, (deg, clamp) in GC.VARIANTS.items():
        coef, _ = header_coeffs(name)
        fitted = GC.fit(deg, clamp)
        np.testing.assert_allclose(fitted, coef, rtol=1e-6, atol=1e-9, err_msg=name)
