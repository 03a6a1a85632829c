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


# A row of the output may fail the gate only where the first layer's scores
# of that query are tied to within fp32 resolution (reading C4 #14 of the
# precision contract: report such rows, never widen the tolerance).  With
# raw inputs near 1e3 the first-layer scores reach ~1e5; when the two best
# keys of a query differ by less than 2^-16 of the score magnitude (a few
# hundred fp32 roundings of the score), the softmax weights of the two keys,
# and through them every later value of the row, depend on the score's last
# bits, which no fp32-accumulated computation resolves: a plain fp32 PyTorch
# evaluation of the same definition fails such rows by more than this path.
NEAR_TIE_REL = 2.0 ** -16


def first_layer_gaps(inp, b: int) -> np.ndarray:
    """For each query i of sequence b: the smallest, over heads, first-layer
    gap between the largest and second-largest score among the keys the
    query may see, relative to the largest score's magnitude (fp64, from the
    oracle's projection of the stored inputs).  inf for a single key."""
    import oracle
    from masked_attention_causal_amd import synth
    w = inp.w
    lw = {k: synth.to_f64(v, w.dtype) for k, v in inp.layers[0].items()}
    qkv = oracle.linear(synth.to_f64(inp.x[b], w.dtype), lw["w_qkv"], lw["b_qkv"])
    d, dh, ln = w.d, w.d // w.H, int(min(max(inp.lens[b], 1), w.L))
    out = np.full(w.L, np.inf)
    for h in range(w.H):
        q = qkv[:, h * dh:(h + 1) * dh]
        k = qkv[:ln, d + h * dh:d + (h + 1) * dh]
        S = q @ k.T / np.sqrt(dh)                    # [L, ln]
        for i in range(w.L):
            s = np.sort(S[i, :min(i, ln - 1) + 1])
            if s.size > 1:
                out[i] = min(out[i], (s[-1] - s[-2]) / max(abs(s[-1]), abs(s[-2])))
    return out


def assert_gate_near_ties(y, ref, inp, what: str = "", max_rows: int = 8) -> dict:
    """The gate on every element, except output rows whose first-layer scores
    are tied to within NEAR_TIE_REL; those are listed, and at most max_rows
    of them may fail."""
    g = gate(y, ref)
    say(f"    gate {what}: n={g['n']} fail={g['fail']} env={g['env']:.4f} rms={g['rms']:.3e}")
    if g["fail"] == 0:
        return g
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    bad = ~(np.abs(y - ref) / np.maximum(ATOL, RTOL * np.abs(ref)) <= 1.0)
    rows = sorted({(int(b), int(i)) for b, i, _ in np.argwhere(bad)})
    gaps = {}
    for b, i in rows:
        if b not in gaps:
            gaps[b] = first_layer_gaps(inp, b)
        r = gaps[b][i]
        n = int(bad[b, i].sum())
        say(f"    failing row (sequence {b}, position {i}, length {int(inp.lens[b])}): {n} elements, "
            f"first-layer relative top-2 score gap {r:.3g}")
        assert r < NEAR_TIE_REL, f"{what}: row ({b}, {i}) fails the gate and its first-layer scores are not tied " \
                                 f"(relative gap {r:.3g})"
    assert len(rows) <= max_rows, f"{what}: {len(rows)} near-tie rows fail"
    say(f"    {len(rows)} row(s) outside the gate, all with first-layer scores tied to within {NEAR_TIE_REL:.3g}")
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
