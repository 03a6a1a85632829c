"""The numerical gate and GPU/oracle runners shared by the tests.

Gate (per element): pass iff |y - o| <= 0.002 OR |y - o| <= 0.02 * |o|, with
o the unrounded fp64 oracle value; NaN or Inf fails.  This is the tolerance
rule of "Hyper-optimized megakernel-hybrid transformer inference",
"Headline results" (atol 0.002 or rtol 0.02), applied to every element.
``env`` is the worst ratio |y - o| / max(0.002, 0.02 |o|); a case passes iff
env <= 1.
"""
from __future__ import annotations

import sys

import numpy as np

ATOL = 0.002
RTOL = 0.02


def gate(y: np.ndarray, ref: np.ndarray) -> dict:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(y - ref)
    env = err / np.maximum(ATOL, RTOL * np.abs(ref))
    env = np.where(np.isfinite(y), env, np.inf)
    worst = int(np.argmax(env)) if env.size else 0
    return {
        "n": int(env.size),
        "fail": int(np.count_nonzero(~(env <= 1.0))),
        "env": float(env.max()) if env.size else 0.0,
        "rms": float(np.sqrt(np.mean(err[np.isfinite(err)] ** 2))) if env.size else 0.0,
        "worst": np.unravel_index(worst, y.shape) if env.size else None,
    }


def assert_gate(y, ref, what: str = "") -> dict:
    g = gate(y, ref)
    say(f"    gate {what}: n={g['n']} fail={g['fail']} env={g['env']:.4f} rms={g['rms']:.3e}")
    assert g["fail"] == 0, f"{what}: {g['fail']}/{g['n']} elements outside the gate, env={g['env']:.3f} at {g['worst']}"
    return g


def say(*a) -> None:
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_forward(inp, eps: float = 1e-5) -> np.ndarray:
    import oracle
    return oracle.forward(inp.x64(), inp.lens, inp.layers64(), inp.w.H, eps)


def gpu_forward(inp, force_path: str = "auto", eps: float = 0.0, return_encoder: bool = False, lib_path=None):
    import torch

    import masked_attention_causal_amd as tfl
    w = inp.w
    layers = [{k: tfl.to_device(v, w.dtype) for k, v in lw.items()} for lw in inp.layers]
    enc = tfl.Encoder(w.n_layers, w.d, w.H, w.f, w.B, w.L, w.dtype, layers, ln_eps=eps, force_path=force_path,
                      lib_path=lib_path or tfl.LIB_PATH)
    x = tfl.to_device(inp.x, w.dtype)
    lens = torch.from_numpy(inp.lens).cuda()
    y = enc.forward(x, lens)
    torch.cuda.synchronize()
    out = tfl.to_numpy_f64(y)
    if return_encoder:
        return out, enc, x, lens
    enc.close()
    return out
