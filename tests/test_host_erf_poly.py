"""The short-range erf polynomial of the fused kernel (common.h, erf_small).

Host-side check of the coefficients the device code uses: evaluated the way
the kernel evaluates them (fp32 Horner in x^2, times x), erf must stay within
3 ulp of math.erf on |x| <= 1, the range the kernel hands it (larger
arguments go to the library erf).  The coefficients are read from the header,
so a typo there fails here.
"""
import math
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HDR = os.path.join(HERE, "..", "masked_attention_causal_amd", "csrc", "common.h")


def _coefficients():
    src = open(HDR).read()
    body = src[src.index("float erf_small(float x)"):]
    body = body[:body.index("return x * q;")]
    nums = [float(v) for v in re.findall(r"(-?\d+\.\d+(?:e-?\d+)?)f", body)]
    # fmaf(t, c5, c4) then fmaf(t, q, c3) ... fmaf(t, q, c0): highest degree first
    return nums[0], nums[1:]


def _erf_small(x):
    top, rest = _coefficients()
    x = np.asarray(x, dtype=np.float32)
    t = (x * x).astype(np.float32)
    q = (t * np.float32(top) + np.float32(rest[0])).astype(np.float32)
    for c in rest[1:]:
        q = (t * q + np.float32(c)).astype(np.float32)
    return (x * q).astype(np.float32)


def test_erf_small_within_3_ulp():
    x = np.linspace(-1.0, 1.0, 40001, dtype=np.float32)
    x = x[x != 0]
    got = _erf_small(x).astype(np.float64)
    ref = np.array([math.erf(float(v)) for v in x])
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got - ref) / ulp) <= 3.0


def test_erf_small_odd_and_exact_at_zero():
    x = np.float32([0.25, 0.5, 0.99])
    assert np.array_equal(_erf_small(-x), -_erf_small(x))
    assert _erf_small(np.float32([0.0]))[0] == 0.0


def test_gelu_small_threshold_inside_fit_range():
    src = open(HDR).read()
    thr = float(re.search(r"GELU_SMALL_MAX = (\d+\.\d+)f", src).group(1))
    assert thr * 0.7071067811865475 <= 1.0
