"""tfl_forward_noalloc (include/tfl.h): the forward on the library's static
device workspace, for callers that cannot allocate.  Through the C ABI, its
output must equal tfl_forward's (same kernels, caller-provided workspace)
bit for bit, on two calls in a row where the second has a smaller input,
for each path that uses a workspace (layer-wise, PQ) and one that needs
none; one case is also gated against the fp64 oracle."""
import numpy as np
import pytest
import torch

import masked_attention_causal_amd as tfl
from masked_attention_causal_amd import synth
from tests.gate import assert_gate, oracle_forward, say

pytestmark = pytest.mark.gpu

W = synth.Workload

PAIRS = [
    ("tiled", W("na_tiled_big", 2, 128, 2, 256, 2, 200, "f16", 1, 200, 1.0),
     W("na_tiled_small", 2, 128, 2, 256, 1, 100, "f16", 1, 100, 1.0)),
    ("tiled", W("na_tiled_f32_big", 2, 64, 4, 128, 3, 150, "f32", 1, 150, 1.0),
     W("na_tiled_f32_small", 2, 64, 4, 128, 2, 70, "f32", 1, 70, 1.0)),
    ("pq", W("na_pq_big", 2, 128, 2, 512, 1, 1000, "f32", 900, 1000, 1.0),
     W("na_pq_small", 2, 128, 2, 512, 1, 300, "f32", 1, 300, 1.0)),
    ("seq", W("na_seq_big", 2, 32, 2, 128, 4, 32, "f32", 1, 32, 1.0),
     W("na_seq_small", 2, 32, 2, 128, 2, 20, "f32", 1, 20, 1.0)),
]


def _both(w, path, seed):
    inp = synth.make_inputs(w, seed)
    layers = [{k: tfl.to_device(v, w.dtype) for k, v in lw.items()} for lw in inp.layers]
    enc = tfl.Encoder(w.n_layers, w.d, w.H, w.f, w.B, w.L, w.dtype, layers, force_path=path)
    assert enc.plan_path == path, enc.plan_name
    assert enc.handle.workspace_bytes <= tfl.binding.STATIC_WORKSPACE_BYTES
    x = tfl.to_device(inp.x, w.dtype)
    lens = torch.from_numpy(inp.lens).cuda()
    st = torch.cuda.current_stream().cuda_stream
    y_ws = enc.forward(x, lens)
    y_na = torch.full_like(x, float("nan"))
    enc.handle.forward_noalloc_raw(x.data_ptr(), lens.data_ptr(), y_na.data_ptr(), st)
    torch.cuda.synchronize()
    out = tfl.to_numpy_f64(y_ws), tfl.to_numpy_f64(y_na)
    enc.close()
    return inp, out


@pytest.mark.parametrize("path,big,small", PAIRS, ids=lambda v: v.name if hasattr(v, "name") else v)
def test_noalloc_matches_forward(path, big, small):
    for k, w in enumerate((big, small)):
        say(f"[noalloc] {path} call {k}: {w.name} B={w.B} L={w.L} ({'larger' if k == 0 else 'smaller'} input)")
        inp, (y_ws, y_na) = _both(w, path, seed=k)
        assert np.isfinite(y_na).all()
        assert np.array_equal(y_ws, y_na), f"{w.name}: {np.count_nonzero(y_ws != y_na)} values differ"
        if k == 1:
            assert_gate(y_na, oracle_forward(inp), f"noalloc {w.name}")
