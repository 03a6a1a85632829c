"""Build libtfl.so (HIP, gfx950) in-tree with hipcc, and its audit copy.

    python -m masked_attention_causal_amd.build

Every translation unit is compiled for gfx950 only.  Packed fp32 VALU
instructions are disabled for device code.

libtfl_audit.so is the same sources built with TFL_AUDIT=1 (attention masks
on every key tile and tile counters; include/tfl_audit.h).  Only the tests
load it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtfl.so")
AUDIT_LIB = os.path.join(PKG, "libtfl_audit.so")

SOURCES = ["tfl_api.hip", "plan.hip", "gemm.hip", "attn.hip", "ln.hip", "seq.hip", "seq_small.hip",
           "pq.hip", "pq_f32.hip", "pq_f16.hip", "pq_bf16.hip", "rowfuse.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


# Per-file extra flags.  attn.hip: MFMA accumulators in VGPRs (the softmax
# reads every score, and AGPR operands would cost a move each way).
# gemm.hip: the same (with AGPR accumulators the compiler copied all of them
# to VGPRs and back at every stage of the K loop).  attn.hip
# and seq.hip: no NaN honouring, so a max over scores needs no quieting pass
# (the kernels never produce NaN from finite inputs; masks use -inf, which is
# still honoured).
EXTRA: dict = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
               "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "seq.hip": ["-fno-honor-nans"]}


def _compile(job) -> str:
    src, objdir, defs = job
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *defs, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, audit: bool = True) -> str:
    """Compiles libtfl.so (and, with audit, libtfl_audit.so) from scratch."""
    variants = [(LIB, os.path.join(BUILD, "product"), [])]
    if audit:
        variants.append((AUDIT_LIB, os.path.join(BUILD, "audit"), ["-DTFL_AUDIT=1"]))
    jobs = []
    for _, objdir, defs in variants:
        os.makedirs(objdir, exist_ok=True)
        jobs += [(src, objdir, defs) for src in SOURCES]
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, jobs))
    for i, (out, _, _) in enumerate(variants):
        _link(objs[i * len(SOURCES):(i + 1) * len(SOURCES)], out)
        if verbose:
            print(f"built {out}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, audit="--no-audit" not in sys.argv)
    sys.exit(0)
