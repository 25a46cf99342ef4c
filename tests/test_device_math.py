"""Constants and algebra of the device-side GELU, checked on the CPU.

The GEMM epilogues evaluate GELU and its derivative through the normal tail
Phi(-|z|) = erfc(|z| / sqrt 2) / 2 taken from Abramowitz & Stegun, Handbook of Mathematical
Functions, formula 7.1.26 (published absolute error bound 1.5e-7 on erf).  These tests read the
coefficients from the device header, check them against the published values, and evaluate the
header's formulas in float64 against scipy, so a mistyped coefficient, a wrong sign or a wrong
fold of 1/sqrt 2 or 1/2 fails here (the kernels themselves are checked against the oracle by the
GPU parity tests).
"""
import os
import re

import numpy as np
from scipy.special import erf

HDR = os.path.join(os.path.dirname(__file__), "..", "mixture_experts_layer_group_amd", "csrc",
                   "moe_device.h")

# Abramowitz & Stegun 7.1.26
P_AS = 0.3275911
A_AS = (0.254829592, -0.284496736, 1.421413741, -1.453152027, 1.061405429)


def _body(name):
    src = open(HDR).read()
    body = src[src.index(name):]
    return body[:body.index("\n}")]


def _tail_constants():
    """(p, scale, (a1..a5) as written before halving, halving factors, exp2 coefficient)."""
    body = _body("float normal_tail_as7126(")
    m = re.search(r"fmaf\(([0-9.]+)f \* ([0-9.]+)f, az, 1\.0f\)", body)
    p, scale = float(m.group(1)), float(m.group(2))
    halved = re.findall(r"(0\.5)f \* (-?[0-9.]+)f", body)
    assert len(halved) == 5
    a5, a4, a3, a2, a1 = (float(v) for _, v in halved)
    halves = {float(h) for h, _ in halved}
    c = float(re.search(r"z \* z \* (-[0-9.]+)f", _body("float exp_neg_half_sq(")).group(1))
    return p, scale, (a1, a2, a3, a4, a5), halves, c


def _tail(z):
    p, scale, (a1, a2, a3, a4, a5), _, c = _tail_constants()
    az = np.abs(z)
    t = 1.0 / (1.0 + p * scale * az)
    e = np.exp2(c * z * z)
    q = 0.5 * t * (a1 + t * (a2 + t * (a3 + t * (a4 + t * a5)))) * e
    return q, e


def test_constants_are_the_published_ones():
    p, scale, a, halves, c = _tail_constants()
    assert p == P_AS and a == A_AS and halves == {0.5}
    assert abs(scale - 2 ** -0.5) < 1e-15
    assert abs(c + 0.5 / np.log(2.0)) < 1e-15


def test_erf_from_the_tail_within_published_bound():
    # erf(x) = 1 - 2 Phi(-sqrt 2 x) for x >= 0, odd extension
    x = np.linspace(-6.0, 6.0, 240001)
    q, _ = _tail(np.sqrt(2.0) * x)
    y = np.sign(x) * (1.0 - 2.0 * q)
    assert np.max(np.abs(y - erf(x))) <= 1.5e-7


def test_gelu_sign_shared_form_within_bound():
    """gelu_erf = max(z, 0) - |z| Phi(-|z|): within |z| / 2 times the erf bound of z Phi(z)."""
    body = _body("float gelu_erf(float z)")
    assert "fmaf(-az, normal_tail_as7126(az, exp_neg_half_sq(z)), fmaxf(z, 0.0f))" in body
    z = np.linspace(-8.0, 8.0, 320001)
    q, _ = _tail(z)
    g = np.maximum(z, 0.0) - np.abs(z) * q
    exact = 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))
    assert np.all(np.abs(g - exact) <= 0.75e-7 * np.abs(z) + 1e-15)


def test_gelu_grad_form_within_bound():
    """gelu_grad = Phi(z) + z phi(z), Phi from the tail (1 - tail for z > 0) and phi sharing its
    exponential: within half the erf bound of the exact derivative."""
    body = _body("float gelu_grad(float z)")
    assert "z > 0.0f ? 1.0f - q : q" in body
    assert "fmaf(z * 0.39894228040143267794f, e, Phi)" in body
    z = np.linspace(-8.0, 8.0, 320001)
    q, e = _tail(z)
    phi_cdf = np.where(z > 0.0, 1.0 - q, q)
    g = phi_cdf + z * 0.39894228040143267794 * e
    exact = 0.5 * (1.0 + erf(z / np.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)
    assert np.max(np.abs(g - exact)) <= 0.75e-7 + 1e-15
