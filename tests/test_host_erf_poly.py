"""The short-range GELU polynomial of the fused kernels (common.h, gelu_poly).

Host-side check of the coefficients the device code uses.  The kernel
computes GELU(h) = h/2 + u R(u), u = h^2, for |h| < GELU_SMALL_MAX, where
R(u) = P(u/2) / (2 sqrt(2)) and erf(x) = x P(x^2) is the degree-5 fit of
csrc/fit_erf_poly.py.  Checked here: the erf polynomial those coefficients
imply stays within 3 ulp of math.erf on |x| <= 1; evaluated the way the
kernel evaluates it (fp32 fused multiply-adds), GELU stays within 11 ulp of
the exact erf-based GELU -- no worse than forming h/2 (1 + erf(h / sqrt(2)))
from a 3-ulp erf, whose cancellation as erf nears -1 costs the same -- and
the threshold keeps the erf argument inside the fitted range.  The
coefficients are read from the header, so a typo there fails here.
"""
import math
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HDR = os.path.join(HERE, "..", "masked_attention_causal_amd", "csrc", "common.h")


def _coefficients():
    """R's coefficients, degree 0..5."""
    src = open(HDR).read()
    body = src[src.index("float gelu_poly(float h)"):]
    body = body[:body.index("return fmaf(u, r, 0.5f * h);")]
    nums = [float(v) for v in re.findall(r"(-?\d+\.\d+(?:e-?\d+)?)f", body)]
    # fmaf(u, r5, r4), then fmaf(u, r, r3) ... fmaf(u, r, r0): highest degree first
    assert len(nums) == 6
    return nums[::-1]


def _fma32(a, b, c):
    """fp32 fused multiply-add: exact product and sum in float64, one rounding."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(np.float32)


def _gelu_poly(h):
    r = _coefficients()
    h = np.asarray(h, dtype=np.float32)
    u = (h * h).astype(np.float32)
    q = _fma32(u, np.float32(r[5]), np.float32(r[4]))
    for c in r[3::-1]:
        q = _fma32(u, q, np.float32(c))
    return _fma32(u, q, (np.float32(0.5) * h).astype(np.float32))


def _threshold():
    return float(re.search(r"GELU_SMALL_MAX = (\d+\.\d+)f", open(HDR).read()).group(1))


def test_implied_erf_within_3_ulp():
    r = _coefficients()
    p = [rk * 2.0 * math.sqrt(2.0) * 2.0 ** k for k, rk in enumerate(r)]
    x = np.linspace(-1.0, 1.0, 40001)
    x = x[x != 0]
    got = x * np.polyval(p[::-1], x * x)
    ref = np.array([math.erf(v) for v in x])
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got - ref) / ulp) <= 3.0


def test_gelu_poly_fp32_within_11_ulp():
    thr = _threshold()
    h = np.linspace(-thr, thr, 200001, dtype=np.float32)
    h = h[h != 0]
    got = _gelu_poly(h).astype(np.float64)
    ref = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in h.astype(np.float64)])
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got - ref) / ulp) <= 11.0
    # away from the cancellation (h > -1) it is a few ulp
    keep = h > -1.0
    assert np.max((np.abs(got - ref) / ulp)[keep]) <= 4.0


def test_gelu_poly_identities():
    h = np.float32([0.125, 0.5, 1.0, 1.375])
    assert _gelu_poly(np.float32([0.0]))[0] == 0.0
    # GELU(h) - GELU(-h) = h
    d = _gelu_poly(h).astype(np.float64) - _gelu_poly(-h).astype(np.float64)
    assert np.allclose(d, h.astype(np.float64), rtol=0, atol=2e-7)


def test_gelu_small_threshold_inside_fit_range():
    assert _threshold() * 0.7071067811865475 <= 1.0
