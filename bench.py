#!/usr/bin/env python3
"""Throughput of the masked post-LN encoder-stack forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one full forward of the layer stack (every layer, every stage)
over one batch of seeded synthetic input already resident in HBM.  The
default workload is the 2-layer, d_model 256, 4-head, FFN 1024, fp16,
batch 4096 x 64-token one with valid lengths uniform in [8, 64].

Prints one JSON line: sequences/s (value), ms per forward, the roofline of
the dominant kernel (its algorithmic bytes or FLOPs per launch over its
average launch time, measured with HIP events on the forward's stream inside
the timed region) and the fp64 CPU oracle timed on a bounded sample of the
same workload on this host's cores.  Beside the headline, "workloads" gives
the same figures (fewer steps, no CPU leg) for the four other named
workloads, and "dispatch" the paths the dispatcher chooses between, timed
in interleaved rounds with rotating order on the workloads where the
choice matters.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
# Transcendental issue: 256 CUs x 4 SIMDs x 32 fp32 lanes per clock (the
# 157.3 TFLOP/s fp32 vector peak over 2 FLOPs per FMA at 2.4 GHz), with
# v_exp_f32 at a quarter of the FMA rate: 1.966e13 exponentials per second.
PEAK_EXP_TPS = 256 * 4 * 32 / 4 * 2.4e9 / 1e12


def allowed_pairs(lens, L):
    """S = sum_b sum_{i<L} min(i+1, len_b): (query, key) pairs that pass the mask."""
    s = 0
    for n in lens:
        n = int(n)
        s += n * (n + 1) // 2 + (L - n) * n
    return s


def stage_work(w, stage, lens):
    """Algorithmic (FLOPs, HBM bytes) of ONE launch of a stage (one layer).
    Operand dtype: fp32 for fp32 I/O, fp16 otherwise; residual, Q and K fp32."""
    T, d, f, H = w.B * w.L, w.d, w.f, w.H
    io = 4 if w.dtype == "f32" else 2
    op = io
    wt = io
    if stage == "prep":
        return 0.0, T * d * (io + 4 + op)
    if stage == "qkv":
        return 2.0 * T * d * 3 * d, T * d * op + 3 * d * d * wt + 2 * T * d * 4 + T * d * op
    if stage == "attn":
        S = allowed_pairs(lens, w.L)
        return 4.0 * d * S, 2 * T * d * 4 + T * d * op + T * d * op + 4 * w.B
    if stage == "out":
        return 2.0 * T * d * d, T * d * op + d * d * wt + 2 * T * d * 4
    if stage == "ln":
        return 0.0, T * d * 4 + T * d * (4 + op)
    if stage == "ffn1":
        return 2.0 * T * d * f, T * d * op + f * d * wt + T * f * op
    if stage == "ffn2":
        return 2.0 * T * f * d, T * f * op + d * f * wt + 2 * T * d * 4
    if stage == "row":
        # fused row kernel of the layer-wise path, per launch (a non-last layer):
        # out-projection, FFN, next layer's QKV; O in, residual in/out twice, Q K V out
        flops = 2.0 * T * d * d + 4.0 * T * d * f + 2.0 * T * d * 3 * d
        nbytes = T * d * op + 4 * T * d * 4 + 3 * T * d * op + (4 * d * d + 2 * d * f) * wt
        return flops, nbytes
    if stage == "fused":
        S = allowed_pairs(lens, w.L)
        flops = w.n_layers * (2.0 * T * d * 3 * d + 4.0 * d * S + 2.0 * T * d * d + 4.0 * T * d * f)
        weights = w.n_layers * (3 * d * d + d * d + 2 * d * f + 6 * d + f) * wt
        return flops, 2 * T * d * io + weights + 4 * w.B
    raise ValueError(stage)


STAGES_TILED = ("prep", "qkv", "attn", "out", "ln", "ffn1", "ffn2")
STAGES_ROWFUSED = ("prep", "qkv", "attn", "row")


def plan_stages(plan, path):
    if path in ("seq", "pq"):
        return ("fused",)
    return STAGES_ROWFUSED if plan.endswith("/rowfused") else STAGES_TILED

def arith_dtype(plan):
    """Operand type the plan's products are computed in (fp16 operands with
    fp32 accumulation, or fp32 throughout)."""
    return "f16" if ("f16op" in plan or "f16x3" in plan) else "f32"


def stage_kernel(stage, plan, w):
    """(kernel name, source files) behind a stage of a plan.  A traffic figure
    taken with rocprofv3 is used only while these files are unchanged."""
    base = ("common.h", "kernels.h")
    if stage == "fused":
        if plan.startswith("SEQ/small"):
            return "seq_small_kernel", ("seq_small.hip",) + base
        if plan.startswith("SEQ"):
            return "seq_kernel", ("seq.hip",) + base
        return "pq_stage_kernel", ("pq_impl.h", "pq.hip") + base
    if stage == "attn":
        return ("attn_ring16_kernel" if w.dh == 16 else "attn_ring_kernel"), ("attn.hip",) + base
    if stage == "row":
        return "row_kernel", ("rowfuse.hip", "pq_impl.h") + base
    if stage in ("qkv", "out", "ffn1", "ffn2"):
        return "gemm_pipe_kernel", ("gemm.hip",) + base
    if stage == "ln":
        return "ln_kernel", ("ln.hip",) + base
    if stage == "prep":
        return "prep_kernel", ("ln.hip",) + base
    return None, ()


def measured_traffic(stage, workload, plan, w):
    """HBM bytes per launch recorded in profiles/*.md for this kernel, stage
    and workload (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the
    kernel's sources changed since the counters were taken or the counters
    are for another stage of the same kernel."""
    import glob
    import hashlib
    kern, files = stage_kernel(stage, plan, w)
    if kern is None:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "masked_attention_causal_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    digest = h.hexdigest()
    for md in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(md) as fh:
            for line in fh:
                if not line.startswith("machine-readable:"):
                    continue
                kv = dict(t.split("=", 1) for t in line.split()[1:] if "=" in t)
                if (kv.get("kernel") == kern and kv.get("workload") == workload
                        and kv.get("stage", stage) == stage
                        and kv.get("source_sha256") == digest and "traffic_bytes_per_launch" in kv):
                    return int(kv["traffic_bytes_per_launch"])
    return None


def launches_per_forward(stage, n_layers, plan=""):
    if stage == "qkv" and plan.endswith("/rowfused"):
        return 1   # later layers' QKV runs inside the fused row kernel
    return {"prep": 1, "ln": 2 * n_layers, "fused": 1}.get(stage, n_layers)


def roofline(w, stage, lens, avg_ms, plan):
    flops, nbytes = stage_work(w, stage, lens)
    peak = PEAK_MFMA_TFLOPS[arith_dtype(plan)]
    t_mfma = flops / (peak * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    sec = avg_ms / 1e3
    # attention also needs one exponential per allowed (query, key) pair and
    # head; at small head dims that, not the products, is the bound
    exps = w.H * allowed_pairs(lens, w.L) if stage == "attn" else 0
    t_exp = exps / (PEAK_EXP_TPS * 1e12)
    if t_exp > max(t_mfma, t_hbm):
        ach = exps / sec / 1e12
        return {"bound": "alu", "achieved": round(ach, 3), "peak": round(PEAK_EXP_TPS, 3), "unit": "Texp/s",
                "frac": round(ach / PEAK_EXP_TPS, 4), "traffic": None, "kernel_stage": stage,
                "avg_launch_us": round(avg_ms * 1e3, 2), "algorithmic_exps_per_launch": exps,
                "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes,
                "mfma_frac": round(flops / sec / 1e12 / peak, 4)}
    if t_mfma >= t_hbm:
        ach = flops / sec / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": None, "kernel_stage": stage,
                "avg_launch_us": round(avg_ms * 1e3, 2), "algorithmic_flops_per_launch": flops,
                "algorithmic_bytes_per_launch": nbytes}
    ach = nbytes / sec / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None, "kernel_stage": stage,
            "avg_launch_us": round(avg_ms * 1e3, 2), "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": nbytes}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, target_s=15.0):
    """The fp64 oracle, as it is, on a bounded sample of the same inputs."""
    import numpy as np

    import oracle
    from masked_attention_causal_amd import synth
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    if w.B == 1:
        if w.L > 8192:
            return None
        t0 = time.perf_counter()
        oracle.forward(inp.x64(), inp.lens, inp.layers64(), w.H)
        dt = time.perf_counter() - t0
        return {"value": round(1.0 / dt, 4), "unit": "sequences/s", "cores": threads, "kind": "oracle",
                "cpu": cpu_model(), "sample": f"the whole batch-1 workload once ({dt:.2f} s)"}
    n0 = min(w.B, 16)
    sub = synth.subset(inp, np.arange(n0))
    t0 = time.perf_counter()
    oracle.forward(sub.x64(), sub.lens, sub.layers64(), w.H)
    dt0 = time.perf_counter() - t0
    n = int(min(w.B, max(n0, n0 * target_s / max(dt0, 1e-3))))
    sub = synth.subset(inp, np.arange(n))
    x64, l64 = sub.x64(), sub.layers64()
    t0 = time.perf_counter()
    oracle.forward(x64, sub.lens, l64, w.H)
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "sequences/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(), "sample": f"first {n} of {w.B} sequences of the same seeded batch, {dt:.1f} s"}


def measure(tfl, torch, w, name, inp, steps, warmup, path="auto"):
    """Warm-up, per-stage survey, then `steps` forwards between HIP events
    with the dominant stage's launches timed as they run; then a separate
    pass of single-forward events for the distribution."""
    layers = [{k: tfl.to_device(v, w.dtype) for k, v in lw.items()} for lw in inp.layers]
    enc = tfl.Encoder(w.n_layers, w.d, w.H, w.f, w.B, w.L, w.dtype, layers, force_path=path)
    x = tfl.to_device(inp.x, w.dtype)
    lens = torch.from_numpy(inp.lens).cuda()
    y = torch.empty_like(x)
    ws = enc.workspace()
    h = enc.handle
    plan = enc.plan_name
    print(f"# workload {name} plan {plan} workspace {h.workspace_bytes / 2**20:.1f} MiB", file=sys.stderr,
          flush=True)

    # first call in this process for this plan, then warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    enc.forward(x, lens, y, ws)
    torch.cuda.synchronize()
    cold_ms = (time.perf_counter() - t0) * 1e3
    for _ in range(warmup):
        enc.forward(x, lens, y, ws)
    torch.cuda.synchronize()

    # per-stage survey (not timed): which kernel dominates the forward
    stages = plan_stages(plan, enc.plan_path)
    survey = {}
    reps = 3 if w.B * w.L < 50000 else 1
    for st in stages:
        per = launches_per_forward(st, w.n_layers, plan)
        h.timer_arm(st, per * reps)
        for _ in range(reps):
            enc.forward(x, lens, y, ws)
        ms, n = h.timer_read()
        survey[st] = ms / reps
    dom = max(survey, key=survey.get)

    # timed region: K steps, dominant stage timed with HIP events as it runs
    per = launches_per_forward(dom, w.n_layers, plan)
    h.timer_arm(dom, per * steps)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        enc.forward(x, lens, y, ws)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    dom_ms, dom_n = h.timer_read()
    ms_step = total_ms / steps
    roof = roofline(w, dom, inp.lens, dom_ms / max(dom_n, 1), plan)
    roof["kernel"] = stage_kernel(dom, plan, w)[0]
    roof["launches_timed"] = dom_n
    roof["traffic"] = measured_traffic(dom, name, plan, w)

    # per-forward distribution, in a pass of its own after the timed region
    # (one event pair per forward; the timed region above has none of these)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(steps):
        enc.forward(x, lens, y, ws)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_us = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps))
    pick = lambda q: round(per_us[min(len(per_us) - 1, int(q * len(per_us)))], 2)
    dist = {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9), "forwards": len(per_us)}

    # whole-forward figure for context
    tot_flops = 0.0
    fstages = ("fused",) if enc.plan_path in ("seq", "pq") else ("qkv", "attn", "out", "ffn1", "ffn2")
    for st in fstages:
        tot_flops += stage_work(w, st, inp.lens)[0] * (1 if st == "fused" else w.n_layers)
    launches = sum(launches_per_forward(st, w.n_layers, plan) for st in stages)
    if enc.plan_path == "pq":
        # QKV, ATT, FFN per layer, the final rows (the first QKV stage also
        # converts the weights)
        launches = 3 * w.n_layers + 1
    res = {
        "plan": plan,
        "ms_per_step": ms_step,
        "sequences_per_s": w.B / (ms_step / 1e3),
        "roofline": roof,
        "forward_tflops": round(tot_flops / (ms_step / 1e3) / 1e12, 2),
        "stage_ms_per_forward": {k: round(v, 4) for k, v in survey.items()},
        "us_per_forward_dist": dist,
        "cold_first_call_ms": round(cold_ms, 2),
        # the layer-wise prep stage also pads V^T and, with bf16 or fp32 I/O,
        # converts the GEMM weights to fp16 planes (one launch per 8 layers)
        "launches_per_forward": launches + ((1 + (0 if w.dtype == "f16" else (w.n_layers + 7) // 8))
                                            if enc.plan_path == "tiled" else 0),
    }
    enc.close()
    return res


def interleaved(tfl, torch, w, inp, paths, rounds=6, iters=5):
    """Median us per forward of each path, timed in rounds of `iters`
    forwards with the order of the paths rotated every round."""
    import numpy as np
    layers = [{k: tfl.to_device(v, w.dtype) for k, v in lw.items()} for lw in inp.layers]
    x = tfl.to_device(inp.x, w.dtype)
    lens = torch.from_numpy(inp.lens).cuda()
    encs = {p: tfl.Encoder(w.n_layers, w.d, w.H, w.f, w.B, w.L, w.dtype, layers, force_path=p) for p in paths}
    ys = {p: torch.empty_like(x) for p in paths}
    for p in paths:
        for _ in range(2):
            encs[p].forward(x, lens, ys[p])
    torch.cuda.synchronize()
    times = {p: [] for p in paths}
    for r in range(rounds):
        order = paths[r % len(paths):] + paths[:r % len(paths)]
        for p in order:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(iters):
                encs[p].forward(x, lens, ys[p])
            b.record()
            torch.cuda.synchronize()
            times[p].append(a.elapsed_time(b) * 1e3 / iters)
    out = {p: {"plan": encs[p].plan_name, "us_median": round(float(np.median(times[p])), 2),
               "us_rounds": [round(v, 1) for v in times[p]]} for p in paths}
    for e in encs.values():
        e.close()
    return out


# Steps and warm-up for the workloads reported beside the headline (the
# 100k-token forward takes ~7 ms, the others well under 1 ms).
EXTRA_STEPS = {"tiny_d32_b4_l32": (300, 30), "gemm_d1024_b8_l512": (40, 5),
               "latency_d128_b1_l4096": (200, 20), "stream_d64_b1_l100000": (10, 2)}
# Workloads whose plan choice is timed against its alternative.
DISPATCH = {"batch4096_d256_l64": ["seq", "tiled"], "latency_d128_b1_l4096": ["pq", "tiled"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--path", default="auto", choices=["auto", "seq", "pq", "tiled"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads and the path comparison")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import torch

    import masked_attention_causal_amd as tfl
    from masked_attention_causal_amd import synth

    name = args.workload or synth.BENCH_WORKLOAD
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w, args.seed)
    torch.cuda.set_device(0)
    m = measure(tfl, torch, w, name, inp, args.steps, args.warmup, args.path)
    ms_step = m["ms_per_step"]

    extra, dispatch = {}, {}
    if not args.no_extra:
        for other, (st, wu) in EXTRA_STEPS.items():
            if other == name:
                continue
            ow = synth.WORKLOADS[other]
            oi = synth.make_inputs(ow, args.seed)
            r = measure(tfl, torch, ow, other, oi, st, wu)
            extra[other] = {"plan": r["plan"], "us_per_forward": round(r["ms_per_step"] * 1e3, 2),
                            "sequences_per_s": round(r["sequences_per_s"], 2), "steps": st,
                            "launches_per_forward": r["launches_per_forward"], "roofline": r["roofline"],
                            "stage_ms_per_forward": r["stage_ms_per_forward"],
                            "us_per_forward_dist": r["us_per_forward_dist"]}
            del oi
        for dn, paths in DISPATCH.items():
            dw = synth.WORKLOADS[dn]
            di = inp if dn == name else synth.make_inputs(dw, args.seed)
            dispatch[dn] = interleaved(tfl, torch, dw, di, paths)

    cpu = None if args.no_cpu else cpu_baseline(w, inp)
    out = {
        "metric": "sequences/s per stack forward (with us per forward and roofline fraction)",
        "value": round(m["sequences_per_s"], 1),
        "unit": "sequences/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_forward": round(ms_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": arith_dtype(m["plan"]),
        "data": "synthetic (seeded normals, weights N(0,0.02^2), random valid lengths)",
        "config": {"workload": name, "io_dtype": w.dtype, "n_layers": w.n_layers, "d_model": w.d, "n_heads": w.H,
                   "d_ffn": w.f, "batch": w.B, "seq_len": w.L, "valid_len": [w.len_lo, w.len_hi],
                   "input_scale": round(inp.scale, 6), "seed": args.seed, "plan": m["plan"],
                   "parallelism": "single GPU"},
        "roofline": m["roofline"],
        "forward_tflops": m["forward_tflops"],
        "stage_ms_per_forward": m["stage_ms_per_forward"],
        "us_per_forward_dist": m["us_per_forward_dist"],
        "cold_first_call_ms": m["cold_first_call_ms"],
        "launches_per_forward": m["launches_per_forward"],
        "cpu_baseline": cpu,
        "workloads": extra,
        "dispatch": dispatch,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
