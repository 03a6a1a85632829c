"""Write stored oracle rows for the 100,000-token workload.

    python tests/golden/make_stream_golden.py

Runs only the fp64 CPU oracle (oracle/) on the seeded inputs of the
2-layer, d_model 64, 4-head, FFN 256, fp16, batch 1, 100,000-token workload
(valid length 99,000, seed 0, input scale 1) and stores a sample of output
rows, including padded rows past the valid length and rows on tile
boundaries.  The whole oracle takes minutes, so the GPU test compares
against these stored values instead of recomputing them.
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from masked_attention_causal_amd import synth  # noqa: E402

ROWS = [0, 1, 2, 15, 16, 63, 64, 65, 127, 128, 4095, 4096, 25000, 50000, 65535, 65536, 77777,
        98998, 98999, 99000, 99500, 99999]


def main():
    w = synth.WORKLOADS["stream_d64_b1_l100000"]
    inp = synth.make_inputs(w, 0, 1.0)
    t0 = time.time()
    y = oracle.forward(inp.x64(), inp.lens, inp.layers64(), w.H)
    dt = time.time() - t0
    out = {
        "workload": w.name, "seed": 0, "scale": 1.0, "lens": inp.lens.tolist(),
        "generator": "masked_attention_causal_amd.synth.make_inputs",
        "oracle_seconds": round(dt, 1), "oracle_threads": oracle.max_threads(),
        "rows": ROWS,
        "values": [[float(v) for v in y[0, r]] for r in ROWS],
    }
    with open(os.path.join(HERE, "stream_d64_l100000_seed0_rows.json"), "w") as fh:
        json.dump(out, fh, indent=0)
    print(f"oracle {dt:.1f} s on {oracle.max_threads()} threads; wrote {len(ROWS)} rows")


if __name__ == "__main__":
    main()
