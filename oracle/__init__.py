"""ctypes wrapper over the fp64 CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU library never
imports, links or runs anything in this folder, and this folder imports
nothing from the GPU library.

Every function takes and returns float64 numpy arrays.  Layer weights are a
dict with the keys ``w_qkv b_qkv w_o b_o ln1_g ln1_b w_1 b_1 w_2 b_2 ln2_g
ln2_b`` in nn.Linear layout ([out, in], row-major).  The arithmetic, and the
passages of the pages each step follows, are stated in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

LAYER_KEYS = ("w_qkv", "b_qkv", "w_o", "b_o", "ln1_g", "ln1_b",
              "w_1", "b_1", "w_2", "b_2", "ln2_g", "ln2_b")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


class _Layer(ctypes.Structure):
    _fields_ = [(k, _dp) for k in LAYER_KEYS]


def build() -> str:
    """Compile liboracle.so with gcc (plain C, fp64, OpenMP, no fast-math)."""
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fopenmp", "-fPIC", "-shared", SRC, "-o", LIB + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_linear.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp]
        L.orc_attention.argtypes = [ctypes.c_int] * 4 + [_ip, _dp, _dp]
        L.orc_attention.restype = ctypes.c_int
        L.orc_layernorm.argtypes = [ctypes.c_long, ctypes.c_int, _dp, _dp, _dp, ctypes.c_double, _dp]
        L.orc_gelu.argtypes = [ctypes.c_long, _dp, _dp]
        L.orc_out_ln.argtypes = [ctypes.c_long, ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp,
                                 ctypes.c_double, _dp, _dp]
        L.orc_ffn_ln.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp,
                                 _dp, _dp, _dp, ctypes.c_double, _dp, _dp, _dp]
        L.orc_forward.argtypes = [ctypes.c_int] * 6 + [ctypes.c_double, ctypes.POINTER(_Layer),
                                                       _dp, _ip, _dp]
        L.orc_forward.restype = ctypes.c_int
        _lib = L
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


def linear(A, W, b=None) -> np.ndarray:
    """Y = A W^T + b over the last axis of A."""
    A, W = _f64(A), _f64(W)
    n_out, n_in = W.shape
    T = A.size // n_in
    Y = np.empty(A.shape[:-1] + (n_out,), np.float64)
    bb = _f64(b) if b is not None else None
    lib().orc_linear(T, n_in, n_out, _p(A), _p(W), _p(bb) if bb is not None else None, _p(Y))
    return Y


def attention(qkv, lens, n_heads: int) -> np.ndarray:
    """qkv: [B, L, 3d] packed projections; returns o [B, L, d]."""
    qkv = _f64(qkv)
    B, L, d3 = qkv.shape
    d = d3 // 3
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    o = np.empty((B, L, d), np.float64)
    rc = lib().orc_attention(B, L, n_heads, d, lens.ctypes.data_as(_ip), _p(qkv), _p(o))
    if rc != 0:
        raise ValueError(f"oracle attention failed (rc={rc}): lengths must lie in [1, L]")
    return o


def layernorm(z, g, b, eps: float = 1e-5) -> np.ndarray:
    z, g, b = _f64(z), _f64(g), _f64(b)
    d = z.shape[-1]
    out = np.empty_like(z)
    lib().orc_layernorm(z.size // d, d, _p(z), _p(g), _p(b), float(eps), _p(out))
    return out


def gelu(h) -> np.ndarray:
    h = _f64(h)
    g = np.empty_like(h)
    lib().orc_gelu(h.size, _p(h), _p(g))
    return g


def out_ln(X, o, w_o, b_o, g, beta, eps: float = 1e-5) -> np.ndarray:
    """X1 = LN(X + o W_o^T + b_o)."""
    X, o, w_o, b_o, g, beta = map(_f64, (X, o, w_o, b_o, g, beta))
    d = X.shape[-1]
    T = X.size // d
    z = np.empty_like(X)
    X1 = np.empty_like(X)
    lib().orc_out_ln(T, d, _p(X), _p(o), _p(w_o), _p(b_o), _p(g), _p(beta), float(eps), _p(z), _p(X1))
    return X1


def ffn_ln(X1, w_1, b_1, w_2, b_2, g, beta, eps: float = 1e-5) -> np.ndarray:
    """X2 = LN(X1 + GELU(X1 W_1^T + b_1) W_2^T + b_2)."""
    X1, w_1, b_1, w_2, b_2, g, beta = map(_f64, (X1, w_1, b_1, w_2, b_2, g, beta))
    d = X1.shape[-1]
    f = w_1.shape[0]
    T = X1.size // d
    hb = np.empty((T, f), np.float64)
    z = np.empty_like(X1)
    X2 = np.empty_like(X1)
    lib().orc_ffn_ln(T, d, f, _p(X1), _p(w_1), _p(b_1), _p(w_2), _p(b_2), _p(g), _p(beta),
                     float(eps), _p(hb), _p(z), _p(X2))
    return X2


def forward(x, lens, layers, n_heads: int, eps: float = 1e-5) -> np.ndarray:
    """Whole stack: x [B, L, d] float64 (values as stored), lens int32 [B],
    layers: list of dicts of float64 arrays.  Returns y [B, L, d] float64."""
    x = _f64(x)
    B, L, d = x.shape
    f = np.asarray(layers[0]["w_1"]).shape[0]
    keep = []
    arr = (_Layer * len(layers))()
    for i, lw in enumerate(layers):
        for k in LAYER_KEYS:
            a = _f64(lw[k])
            keep.append(a)
            setattr(arr[i], k, _p(a))
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    y = np.empty_like(x)
    rc = lib().orc_forward(len(layers), d, n_heads, f, B, L, float(eps), arr, _p(x),
                           lens.ctypes.data_as(_ip), _p(y))
    if rc != 0:
        raise ValueError(f"oracle forward failed (rc={rc})")
    return y
