"""The GELU forms of the kernels (common.h: gelu_poly, gelu_poly16, gelu_full).

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
import pytest

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


# ---------------------------------------------------------------- short range, fp16 outputs (gelu_poly16)

def _coefficients16():
    """gelu_poly16's R, degree 0..3, read from the header."""
    src = open(HDR).read()
    body = src[src.index("float gelu_poly16(float h)"):]
    body = body[:body.index("return fmaf(u, r, 0.5f * h);")]
    nums = [float(v) for v in re.findall(r"(-?\d+\.\d+(?:e-?\d+)?)f", body)]
    assert len(nums) == 4, nums
    return nums[::-1]


def _gelu_poly16(h):
    r = _coefficients16()
    h = np.asarray(h, dtype=np.float32)
    u = (h * h).astype(np.float32)
    q = _fma32(u, np.float32(r[3]), np.float32(r[2]))
    for c in r[1::-1]:
        q = _fma32(u, q, np.float32(c))
    return _fma32(u, q, (np.float32(0.5) * h).astype(np.float32))


def test_gelu_poly16_within_a_fraction_of_an_fp16_ulp():
    """Evaluated in fp32 as the kernels do: within 2e-5 of the exact GELU and
    under 0.75 fp16 ulp of its value (the output is rounded to fp16 next),
    over the short range; the implied erf(x)/x is within 3e-5 relative."""
    thr = _threshold()
    h = np.linspace(-thr, thr, 200001, dtype=np.float32)
    got = _gelu_poly16(h).astype(np.float64)
    ref = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in h.astype(np.float64)])
    err = np.abs(got - ref)
    assert err.max() <= 2e-5
    ulp16 = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    assert np.max(err / ulp16) <= 0.75
    r = _coefficients16()
    p = [rk * 2.0 * math.sqrt(2.0) * 2.0 ** k for k, rk in enumerate(r)]
    x = np.linspace(1e-3, 1.0, 20001)
    rel = np.abs(np.polyval(p[::-1], x * x) - np.array([math.erf(v) / v for v in x])) / np.array([math.erf(v) / v for v in x])
    assert rel.max() <= 3e-5


def test_gelu_poly16_identities():
    h = np.float32([0.125, 0.5, 1.0, 1.375])
    assert _gelu_poly16(np.float32([0.0]))[0] == 0.0
    d = _gelu_poly16(h).astype(np.float64) - _gelu_poly16(-h).astype(np.float64)
    assert np.allclose(d, h.astype(np.float64), rtol=0, atol=2e-7)


# ---------------------------------------------------------------- whole-range form (gelu_full)

def _full_coefficients():
    """gelu_full's R, degree 0..9, read from the header."""
    src = open(HDR).read()
    body = src[src.index("float gelu_full(float h)"):]
    body = body[:body.index("const float e = ")]
    nums = [float(v) for v in re.findall(r"(-?\d+\.\d+(?:e-?\d+)?)f", body)]
    # 1/sqrt(2), 2.0, then fmaf(u, c9, c8), fmaf(u, r, c7) ... fmaf(u, r, c0)
    assert len(nums) == 2 + 10, nums
    return nums[2:][::-1]


def _gelu_full(h, ulp_rcp=0, ulp_exp=0):
    """The kernel's arithmetic in fp32: fused multiply-adds rounded once, the
    reciprocal and exp2 correctly rounded and then moved by ulp_rcp / ulp_exp
    ulps (the hardware instructions are within one ulp)."""
    c = _full_coefficients()
    h = np.asarray(h, dtype=np.float32)
    a = (np.abs(h) * np.float32(0.70710678118654752)).astype(np.float32)
    u = (1.0 / (a + np.float32(2.0)).astype(np.float64)).astype(np.float32)
    for _ in range(abs(ulp_rcp)):
        u = np.nextafter(u, np.float32(np.inf if ulp_rcp > 0 else 0)).astype(np.float32)
    r = _fma32(u, np.float32(c[9]), np.float32(c[8]))
    for k in range(7, -1, -1):
        r = _fma32(u, r, np.float32(c[k]))
    arg = _fma32((a * a).astype(np.float32), np.float32(-1.4426950408889634), r)
    ex = np.exp2(arg.astype(np.float64)).astype(np.float32)
    ex = np.where(ex < np.float32(2.0 ** -126), np.float32(0), ex)      # exp2 flushes denormal results
    for _ in range(abs(ulp_exp)):
        ex = np.nextafter(ex, np.float32(np.inf if ulp_exp > 0 else 0)).astype(np.float32)
    e = (u * ex).astype(np.float32)
    he = (h * e).astype(np.float32)
    return np.where(h >= 0, (h - he).astype(np.float32), he)


def _gelu_ref(h):
    return np.array([0.5 * v * math.erfc(-v / math.sqrt(2.0)) for v in np.asarray(h, np.float64)])


@pytest.mark.parametrize("ulp_rcp,ulp_exp", [(0, 0), (1, 1), (-1, -1), (1, -1)])
def test_gelu_full_error_bounds(ulp_rcp, ulp_exp):
    h = np.concatenate([np.linspace(-13.0, 13.0, 130001), np.linspace(-1e-3, 1e-3, 2001)]).astype(np.float32)
    got = _gelu_full(h, ulp_rcp, ulp_exp).astype(np.float64)
    ref = _gelu_ref(h)
    assert np.max(np.abs(got - ref)) <= 3e-7
    mid = (np.abs(h) <= 3.0) & (ref != 0)
    assert np.max(np.abs(got - ref)[mid] / np.abs(ref[mid])) <= 2e-6


def test_gelu_full_implied_erfc():
    # erfc(a) = 2e for a in [0, 6]: the fit itself, relative 5e-7
    c = _full_coefficients()
    a = np.linspace(0.0, 6.0, 6001)
    u = 1.0 / (2.0 + a)
    r = np.polyval(c[::-1], u)
    got = 2.0 * u * np.exp2(r - a * a * 1.4426950408889634)
    ref = np.array([math.erfc(v) for v in a])
    assert np.max(np.abs(got - ref) / ref) <= 5e-7


def test_gelu_full_identities_and_limits():
    h = np.float32([0.125, 0.5, 1.0, 2.5, 4.0, 7.0])
    assert _gelu_full(np.float32([0.0]))[0] == 0.0
    d = _gelu_full(h).astype(np.float64) - _gelu_full(-h).astype(np.float64)
    assert np.allclose(d, h.astype(np.float64), rtol=0, atol=1e-6)
    big = np.float32([9.5, 13.0, 30.0, 1e4])
    assert np.array_equal(_gelu_full(big), big)          # h e is below half an ulp of h
    huge = np.float32([13.5, 30.0, 1e4])                 # a > 9.3: erfc(a)/2 < 2^-126, flushed
    assert np.all(_gelu_full(-huge) == 0.0)
