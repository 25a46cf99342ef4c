"""Constants of the device-side erf approximation, checked on the CPU.

The GEMM epilogues evaluate GELU with erf from Abramowitz & Stegun, Handbook of Mathematical
Functions, formula 7.1.26, whose published absolute error bound is 1.5e-7.  This test reads
the coefficients from the device header and evaluates the same formula in float64 against
scipy's erf, so a mistyped coefficient or a wrong sign fails here (the kernels themselves are
checked against the oracle by the GPU parity tests).
"""
import os
import re

import numpy as np
from scipy.special import erf

HDR = os.path.join(os.path.dirname(__file__), "..", "mixture_experts_layer_group_amd", "csrc",
                   "moe_device.h")


def _coefficients():
    src = open(HDR).read()
    body = src[src.index("float erf_as7126(float x)"):]
    body = body[:body.index("}")]
    p = float(re.search(r"fmaf\(([0-9.]+)f, ax, 1\.0f\)", body).group(1))
    fm = re.findall(r"fmaf\((?:p|[0-9.]+f), t, (-?[0-9.]+)f\)", body)
    a5 = float(re.search(r"fmaf\(([0-9.]+)f, t,", body).group(1))
    a4, a3, a2, a1 = (float(v) for v in fm)
    return p, (a1, a2, a3, a4, a5)


def test_erf_as7126_within_published_bound():
    p, (a1, a2, a3, a4, a5) = _coefficients()
    x = np.linspace(-6.0, 6.0, 240001)
    ax = np.abs(x)
    t = 1.0 / (1.0 + p * ax)
    poly = t * (a1 + t * (a2 + t * (a3 + t * (a4 + t * a5))))
    y = np.sign(x) * (1.0 - poly * np.exp(-ax * ax))
    assert np.max(np.abs(y - erf(x))) <= 1.5e-7
    assert (p, a1, a5) == (0.3275911, 0.254829592, 1.061405429)
