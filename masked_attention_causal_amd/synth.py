"""Seeded synthetic inputs for the masked post-LN encoder stack.

This module only draws random numbers and stores them in the I/O dtype.  It
holds none of the layer's arithmetic, so both the GPU path and the CPU
oracle may read what it produces.

The workloads stand in for the project pages' benchmark shapes, which the
pages do not print.  Their envelope is given in "KernelForge", "Why it
matters": 2-4 layers, d_model 32-1024, batch 1 to 10,000, sequences 32 to
100,000 tokens, causal masking with a padding mask throughout.  The input
scale sweep 1e-3 .. 1e3 is the one of "Hyper-optimized megakernel-hybrid
transformer inference", "Headline results".

Draw order (numpy PCG64 seeded with ``seed``):
  1. the input scale, when the workload draws it log-uniformly;
  2. x: B*L*d standard normals, times the scale;
  3. lens: integers uniform on [len_lo, len_hi];
  4. per layer: w_qkv, w_o, w_1, w_2 ~ N(0, 0.02^2);
  5. with ``affine=True`` only, per layer: biases ~ N(0, 0.02^2),
     LayerNorm gamma ~ N(1, 0.1^2), beta ~ N(0, 0.1^2).
Without ``affine`` the biases are 0, gamma is 1 and beta is 0.
Every array is rounded once to the I/O dtype (round to nearest even).
bf16 arrays are returned as their raw uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

DTYPES = ("f32", "f16", "bf16")
LAYER_KEYS = ("w_qkv", "b_qkv", "w_o", "b_o", "ln1_g", "ln1_b",
              "w_1", "b_1", "w_2", "b_2", "ln2_g", "ln2_b")


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    d: int
    H: int
    f: int
    B: int
    L: int
    dtype: str
    len_lo: int
    len_hi: int
    scale: float | None          # None: drawn log-uniform on [1e-3, 1e3]

    @property
    def dh(self) -> int:
        return self.d // self.H

    def with_batch(self, B: int) -> "Workload":
        return replace(self, B=B)

    def with_len(self, L: int) -> "Workload":
        return replace(self, L=L, len_lo=min(self.len_lo, L), len_hi=min(self.len_hi, L))


WORKLOADS = {
    w.name: w for w in (
        Workload("tiny_d32_b4_l32", 2, 32, 2, 128, 4, 32, "f32", 1, 32, 1.0),
        Workload("batch4096_d256_l64", 2, 256, 4, 1024, 4096, 64, "f16", 8, 64, None),
        Workload("gemm_d1024_b8_l512", 4, 1024, 16, 4096, 8, 512, "bf16", 256, 512, 1.0),
        Workload("latency_d128_b1_l4096", 2, 128, 2, 512, 1, 4096, "f32", 4000, 4000, 1.0),
        Workload("stream_d64_b1_l100000", 2, 64, 4, 256, 1, 100000, "f16", 99000, 99000, 1.0),
    )
}
BENCH_WORKLOAD = "batch4096_d256_l64"


def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    """Store float64 values in ``dtype`` (round to nearest even)."""
    a = np.asarray(a, dtype=np.float64)
    if dtype == "f32":
        return a.astype(np.float32)
    if dtype == "f16":
        return a.astype(np.float16)
    if dtype == "bf16":
        u = a.astype(np.float32).view(np.uint32).astype(np.uint64)
        lsb = (u >> 16) & 1
        r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
        nan = np.isnan(a)
        if nan.any():
            r[nan] = 0x7FC0
        return r
    raise ValueError(dtype)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of an array stored in ``dtype``."""
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a).astype(np.float64)


@dataclass
class Inputs:
    w: Workload
    seed: int
    scale: float
    x: np.ndarray                 # [B, L, d] stored dtype
    lens: np.ndarray              # [B] int32
    layers: list                  # list of dict name -> stored array

    def x64(self) -> np.ndarray:
        return to_f64(self.x, self.w.dtype)

    def layers64(self) -> list:
        return [{k: to_f64(v, self.w.dtype) for k, v in lw.items()} for lw in self.layers]


def make_inputs(w: Workload, seed: int, scale: float | None = None,
                affine: bool = False, lens=None) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    if scale is None:
        scale = w.scale if w.scale is not None else float(10.0 ** rng.uniform(-3.0, 3.0))
    x = round_to(rng.standard_normal((w.B, w.L, w.d)) * scale, w.dtype)
    drawn = rng.integers(w.len_lo, w.len_hi + 1, size=w.B).astype(np.int32)
    lens = drawn if lens is None else np.ascontiguousarray(lens, dtype=np.int32)
    d, f = w.d, w.f
    layers = []
    for _ in range(w.n_layers):
        lw = {
            "w_qkv": rng.standard_normal((3 * d, d)) * 0.02,
            "w_o": rng.standard_normal((d, d)) * 0.02,
            "w_1": rng.standard_normal((f, d)) * 0.02,
            "w_2": rng.standard_normal((d, f)) * 0.02,
        }
        layers.append(lw)
    for lw in layers:
        if affine:
            lw["b_qkv"] = rng.standard_normal(3 * d) * 0.02
            lw["b_o"] = rng.standard_normal(d) * 0.02
            lw["b_1"] = rng.standard_normal(f) * 0.02
            lw["b_2"] = rng.standard_normal(d) * 0.02
            lw["ln1_g"] = 1.0 + rng.standard_normal(d) * 0.1
            lw["ln1_b"] = rng.standard_normal(d) * 0.1
            lw["ln2_g"] = 1.0 + rng.standard_normal(d) * 0.1
            lw["ln2_b"] = rng.standard_normal(d) * 0.1
        else:
            lw["b_qkv"] = np.zeros(3 * d)
            lw["b_o"] = np.zeros(d)
            lw["b_1"] = np.zeros(f)
            lw["b_2"] = np.zeros(d)
            lw["ln1_g"] = np.ones(d)
            lw["ln1_b"] = np.zeros(d)
            lw["ln2_g"] = np.ones(d)
            lw["ln2_b"] = np.zeros(d)
    stored = [{k: round_to(lw[k], w.dtype) for k in LAYER_KEYS} for lw in layers]
    return Inputs(w=w, seed=seed, scale=float(scale), x=x, lens=lens, layers=stored)


def subset(inp: Inputs, rows) -> Inputs:
    """The same inputs restricted to the sequences ``rows`` (batch independence)."""
    rows = np.asarray(rows)
    return Inputs(w=inp.w.with_batch(len(rows)), seed=inp.seed, scale=inp.scale,
                  x=np.ascontiguousarray(inp.x[rows]), lens=np.ascontiguousarray(inp.lens[rows]),
                  layers=inp.layers)


def prefix(inp: Inputs, n: int) -> Inputs:
    """The first ``n`` positions of every sequence, lengths clipped to ``n``.
    Under causal masking the first n output rows depend on nothing else."""
    return Inputs(w=inp.w.with_len(n), seed=inp.seed, scale=inp.scale,
                  x=np.ascontiguousarray(inp.x[:, :n]),
                  lens=np.minimum(inp.lens, n).astype(np.int32), layers=inp.layers)
