"""Coefficients of the short-range GELU polynomial in common.h (gelu_poly).

erf(x) = x * P(x^2) on |x| <= 1, P of degree 5; the kernel evaluates
GELU(h) = h/2 + u R(u), u = h^2, R(u) = P(u/2) / (2 sqrt(2)), so it prints
both P and R (coefficient k of R is that of P times 2^-k / (2 sqrt(2))).  The coefficients come from
an iteratively reweighted least-squares fit of erf(x)/x against x^2 on 400
Chebyshev nodes that drives down the largest relative error (about 4e-8 in
exact arithmetic); evaluated by Horner's rule in fp32 the result stays within
2.2 ulp of erf.

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


if __name__ == "__main__":
    c, rel = fit()
    print("erf coefficients P (degree 0..5):", ", ".join(f"{float(np.float32(v))!r}f" for v in c))
    r = [v / (2 * math.sqrt(2) * 2 ** k) for k, v in enumerate(c)]
    print("GELU coefficients R (degree 0..5):", ", ".join(f"{np.float32(v)}f" for v in r))
    print(f"max relative error (exact arithmetic) {rel:.3g}; fp32 Horner {fp32_ulp_error(c):.2f} ulp")
