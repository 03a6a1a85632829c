"""Coefficients of the GELU forms in common.h (gelu_poly, gelu_full).

gelu_poly (short range, |h| < sqrt(2)):

erf(x) = x * P(x^2) on |x| <= 1, P of degree 5; the kernel evaluates
GELU(h) = h/2 + u R(u), u = h^2, R(u) = P(u/2) / (2 sqrt(2)), so it prints
both P and R (coefficient k of R is that of P times 2^-k / (2 sqrt(2))).  The coefficients come from
an iteratively reweighted least-squares fit of erf(x)/x against x^2 on 400
Chebyshev nodes that drives down the largest relative error (about 4e-8 in
exact arithmetic); evaluated by Horner's rule in fp32 the result stays within
2.2 ulp of erf.

gelu_poly16 (the same form with P of degree 3, for products whose GELU
output is rounded to fp16): the same fit with deg=3; relative error of
erf(x)/x about 2.8e-5, GELU within 1.7e-5 absolute and under 0.7 fp16 ulp
of its value on |h| < sqrt(2).

gelu_full (whole range, no branch): erfc(a)/2 = u 2^(R(u) - a^2 log2 e) with
a = |h|/sqrt(2) and u = 1/(2 + a), so GELU(h) = h - h e for h >= 0 and h e
for h < 0, e = erfc(a)/2.  R (degree 9 in u) is the same kind of
reweighted least-squares fit of log2(erfc(a)/(2u)) + a^2 log2 e on 2000
Chebyshev nodes of u over a in [0, 9.3] (past 9.3, erfc(a)/2 < 2^-126 and the
hardware exp2 flushes it to 0); its largest error is ~6e-8 in the exponent.

    python masked_attention_causal_amd/csrc/fit_erf_poly.py
"""
import math

import numpy as np


def fit(deg: int = 5, nodes: int = 400, iters: int = 60):
    t = np.array([0.5 - 0.5 * math.cos(math.pi * (k + 0.5) / nodes) for k in range(nodes)])
    x = np.sqrt(t)
    f = np.array([math.erf(v) / v for v in x])
    w = np.ones_like(t)
    V = np.vander(t, deg + 1, increasing=True)
    for _ in range(iters):
        c, *_ = np.linalg.lstsq(V * w[:, None], f * w, rcond=None)
        err = (V @ c - f) / f
        w = w * (1 + 5 * np.abs(err) / np.max(np.abs(err)))
        w /= w.mean()
    return c, float(np.max(np.abs(err)))


def fp32_ulp_error(c):
    c32 = np.asarray(c, dtype=np.float32)
    x = np.linspace(1e-4, 1.0, 20001, dtype=np.float32)
    t = x * x
    q = np.full_like(t, c32[-1])
    for k in range(len(c32) - 2, -1, -1):
        q = (q * t + c32[k]).astype(np.float32)
    e = (x * q).astype(np.float32)
    ref = np.array([math.erf(float(v)) for v in x])
    return float(np.max(np.abs(e.astype(np.float64) - ref) / np.spacing(ref.astype(np.float32))))


LOG2E = 1.4426950408889634
A_MAX = 9.3


def _tail_target(u):
    a = 1.0 / u - 2.0
    return math.log2(math.erfc(a) / (2.0 * u)) + a * a * LOG2E


def fit_tail(deg: int = 9, nodes: int = 2000, iters: int = 80):
    umin = 1.0 / (2.0 + A_MAX)
    k = np.arange(nodes)
    u = umin + (0.5 - umin) * (0.5 - 0.5 * np.cos(np.pi * (k + 0.5) / nodes))
    f = np.array([_tail_target(v) for v in u])
    w = np.ones_like(u)
    V = np.vander(u, deg + 1, increasing=True)
    for _ in range(iters):
        c, *_ = np.linalg.lstsq(V * w[:, None], f * w, rcond=None)
        err = V @ c - f
        w = w * (1 + 5 * np.abs(err) / np.max(np.abs(err)))
        w /= w.mean()
    return c, float(np.max(np.abs(err)))


if __name__ == "__main__":
    c, rel = fit()
    print("erf coefficients P (degree 0..5):", ", ".join(f"{float(np.float32(v))!r}f" for v in c))
    r = [v / (2 * math.sqrt(2) * 2 ** k) for k, v in enumerate(c)]
    print("GELU coefficients R (degree 0..5):", ", ".join(f"{np.float32(v)}f" for v in r))
    print(f"max relative error (exact arithmetic) {rel:.3g}; fp32 Horner {fp32_ulp_error(c):.2f} ulp")
    c3, rel3 = fit(3)
    r3 = [v / (2 * math.sqrt(2) * 2 ** k) for k, v in enumerate(c3)]
    print("gelu_poly16 coefficients R (degree 0..3):", ", ".join(f"{float(np.float32(v))!r}f" for v in r3))
    print(f"max relative error of erf(x)/x (exact arithmetic) {rel3:.3g}")
    t, terr = fit_tail()
    print("gelu_full coefficients R (degree 0..9):", ", ".join(f"{float(np.float32(v))!r}f" for v in t))
    print(f"max exponent error (exact arithmetic) {terr:.3g}")
