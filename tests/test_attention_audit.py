"""Two statements of "KernelForge", "Challenges" about a causal attention
loop, checked on the GPU against the audit build of the library
(libtfl_audit.so: the same sources compiled with TFL_AUDIT=1, see
include/tfl_audit.h).

1. Masking only the key tiles that reach past the diagonal (here also past
   the padding boundary) is bit-identical to masking every tile: the audit
   build masks every tile it visits, and its outputs must equal the product
   build's exactly, on every attention kernel (layer-wise kernels at head
   dims 16, 32 and 64 with single and split scores, the fused SEQ kernel, the
   PQ split-K tasks).
2. A causal loop visits only the key tiles that hold an allowed key.  The
   allowed keys of a block of queries q0 .. q_end-1 of sequence b are
   0 .. min(q_end, len_b) - 1, so a block visits ceil(min(q_end, len_b) / BK)
   key tiles of BK keys; at full length (len_b = L = M tiles) a (sequence,
   head) visits 1 + 2 + ... + M = M(M+1)/2 of the M^2 tiles, the floor
   (M+1)/2M of the pages.  The audit build counts the tiles its kernels
   visit, per workgroup (tiles staged) and per 16-query wave (tiles scored),
   and the counts must equal these sums exactly.

The small fused kernel scores key by key with no tiles and is not audited.
"""
import numpy as np
import pytest

from masked_attention_causal_amd import synth
from tests.gate import say

pytestmark = pytest.mark.gpu

W = synth.Workload
SLOTS = {"tiled_wg": 0, "tiled_wave": 1, "seq_wave": 2, "pq_wg": 3, "pq_wave": 4, "split_wg": 5, "bounded_wg": 6}
# per-workgroup score-variant counts of the layer-wise and PQ attention
# (checked by test_score_variant_follows_magnitude and
# test_pq_score_variant_follows_magnitude, not by the tile-count test)
VARIANT_SLOTS = {"split_wg", "bounded_wg"}


def cdiv(a, b):
    return -(-a // b)


def blocks_sum(lens, L, block, waves_of, kt):
    """Sum over sequences and query blocks of `block` queries of
    ceil(min(q_end, len) / kt), for the whole block and for each 16-query
    wave inside it."""
    wg = wave = 0
    for ln in lens:
        for q0 in range(0, L, block):
            wg += cdiv(min(q0 + block, ln), kt)
            for wv in range(waves_of):
                wave += cdiv(min(q0 + 16 * wv + 16, ln), kt)
    return wg, wave


def expected(w, path, lens):
    per = w.H * w.n_layers
    if path == "tiled":
        block, kt = (128, 128) if w.dh == 16 else (64, 64)
        wg, wave = blocks_sum(lens, w.L, block, block // 16, kt)
        return {"tiled_wg": wg * per, "tiled_wave": wave * per}
    if path == "seq":
        # one 16-query wave per 16 positions of a 64-token slot, 32-key chunks
        _, wave = blocks_sum(lens, 64, 64, 4, 32)
        return {"seq_wave": wave * per}
    if path == "pq":
        # split-K tasks over 64-key tiles: the splits of a query tile together
        # visit the tiles the unsplit loop would
        wg, wave = blocks_sum(lens, w.L, 64, 4, 64)
        return {"pq_wg": wg * per, "pq_wave": wave * per}
    raise ValueError(path)


def run(inp, path, lib_path, counters=None):
    import torch

    import masked_attention_causal_amd as tfl
    w = inp.w
    layers = [{k: tfl.to_device(v, w.dtype) for k, v in lw.items()} for lw in inp.layers]
    enc = tfl.Encoder(w.n_layers, w.d, w.H, w.f, w.B, w.L, w.dtype, layers, force_path=path, lib_path=lib_path)
    assert enc.plan_path == path, enc.plan_name
    x = tfl.to_device(inp.x, w.dtype)
    lens = torch.from_numpy(inp.lens).cuda()
    lib = tfl.load_library(lib_path)
    if counters is not None:
        assert lib.tfl_audit_attach(counters.data_ptr()) == 0
    try:
        y = enc.forward(x, lens)
        torch.cuda.synchronize()
    finally:
        if counters is not None:
            lib.tfl_audit_attach(None)
    out = tfl.to_numpy_f64(y)
    enc.close()
    return out


CASES = [
    # (workload, path, lens): ragged lengths, length 1, full length
    (W("a_tiled_f16_dh64", 2, 128, 2, 256, 3, 300, "f16", 1, 300, 1.0), "tiled", [300, 1, 173]),
    (W("a_tiled_bf16_dh32", 2, 128, 4, 256, 2, 200, "bf16", 1, 200, 1.0), "tiled", [137, 200]),
    (W("a_tiled_f16_dh16", 2, 64, 4, 128, 2, 600, "f16", 1, 600, 1.0), "tiled", [600, 257]),
    (W("a_tiled_bf16_dh16", 1, 64, 4, 128, 2, 300, "bf16", 1, 300, 1.0), "tiled", [1, 300]),
    (W("a_tiled_f32_dh64", 2, 128, 2, 256, 2, 150, "f32", 1, 150, 1.0), "tiled", [150, 64]),
    (W("a_tiled_f32_dh16", 1, 64, 4, 128, 2, 130, "f32", 1, 130, 1.0), "tiled", [129, 130]),
    (W("a_tiled_f32_dh32", 2, 128, 4, 256, 2, 200, "f32", 1, 200, 1.0), "tiled", [200, 71]),
    (W("a_seq_f16_d128_dh64", 2, 128, 2, 256, 5, 64, "f16", 1, 64, 1.0), "seq", [64, 1, 33, 31, 17]),
    (W("a_seq_bf16_d256_dh32", 2, 256, 8, 256, 3, 50, "bf16", 1, 50, 1.0), "seq", [50, 32, 9]),
    (W("a_pq_f32_d128_dh64", 2, 128, 2, 512, 2, 1000, "f32", 1, 1000, 1.0), "pq", [1000, 555]),
    (W("a_pq_bf16_d64_dh32", 2, 64, 2, 128, 1, 700, "bf16", 1, 700, 1.0), "pq", [640]),
]


@pytest.mark.parametrize("w,path,lens", CASES, ids=lambda c: c.name if hasattr(c, "name") else None)
def test_mask_every_tile_is_bit_identical_and_tiles_match(w, path, lens):
    import torch

    import masked_attention_causal_amd as tfl
    inp = synth.make_inputs(w, 4, lens=np.array(lens, np.int32))
    say(f"[audit] {w.name} path={path} lens={lens}: product build")
    y = run(inp, path, tfl.LIB_PATH)
    counters = torch.zeros(8, dtype=torch.int64, device="cuda")
    say(f"[audit] {w.name}: audit build (mask on every tile, tile counters)")
    y_all = run(inp, path, tfl.AUDIT_LIB_PATH, counters)
    assert np.isfinite(y).all()
    assert np.array_equal(y, y_all), f"{w.name}: masking every tile changed {np.count_nonzero(y != y_all)} values"
    got = counters.cpu().numpy()
    want = expected(w, path, lens)
    say(f"[audit] {w.name}: counted {got[:5].tolist()} expected {want}")
    for slot, n in want.items():
        assert int(got[SLOTS[slot]]) == n, (slot, int(got[SLOTS[slot]]), n)
    for slot in set(SLOTS) - set(want) - (VARIANT_SLOTS if path in ("tiled", "pq") else set()):
        assert got[SLOTS[slot]] == 0, slot


@pytest.mark.parametrize("dh,dtype", [(64, "f16"), (16, "f16"), (64, "f32")])
def test_full_length_visits_triangle(dh, dtype):
    """len_b = L = M key tiles: each (sequence, head, layer) stages exactly
    M(M+1)/2 of the M^2 tiles."""
    import torch

    import masked_attention_causal_amd as tfl
    H = 64 // dh if dh < 64 else 2
    d = dh * H
    block = 128 if dh == 16 else 64
    M = 6
    L = M * block
    w = W(f"a_full_dh{dh}_{dtype}", 1, d, H, 128, 2, L, dtype, L, L, 1.0)
    inp = synth.make_inputs(w, 5)
    assert (inp.lens == L).all()
    counters = torch.zeros(8, dtype=torch.int64, device="cuda")
    say(f"[audit full] {w.name} L={L} M={M}")
    run(inp, "tiled", tfl.AUDIT_LIB_PATH, counters)
    wg = int(counters.cpu().numpy()[SLOTS["tiled_wg"]])
    assert wg == w.B * w.H * w.n_layers * M * (M + 1) // 2, wg


@pytest.mark.parametrize("dh", [16, 64])
def test_score_variant_follows_magnitude(dh):
    """Each layer-wise attention workgroup picks its score variant from the
    largest |q_i| and |k_j| of its (sequence, head).  Split: with 16-bit I/O
    the first layer's scores take the hi/lo split only where the bound on a
    single fp16 pass's score error exceeds 2^-8 in exp2 units.  Bounded: when
    every score is within +-14 in exp2 units the weights take no reference.
    The statistics are formed for the first layer and, at head dim 16, for
    every layer (a layer without them neither splits nor bounds).  Inputs of
    scale 1 (|q|, |k| ~ 1): no split, every workgroup with statistics
    bounded.  Scale 1e3: every first-layer workgroup splits and is not
    bounded; the second layer (LayerNorm-bounded input) is bounded where it
    has statistics.  The outputs meet the gate against the oracle."""
    import torch

    import masked_attention_causal_amd as tfl
    from tests.gate import assert_gate, oracle_forward
    H = 4 if dh == 16 else 2
    w = W(f"a_adapt_dh{dh}", 2, dh * H, H, 256, 2, 300, "f16", 1, 300, 1.0)
    bq = 128 if dh == 16 else 64
    layer0_wgs = w.B * w.H * cdiv(w.L, bq)
    later = layer0_wgs if dh == 16 else 0      # second-layer workgroups with statistics
    for scale, want_split, want_bounded in ((1.0, 0, layer0_wgs + later), (1e3, layer0_wgs, later)):
        inp = synth.make_inputs(w, 7, scale=scale)
        counters = torch.zeros(8, dtype=torch.int64, device="cuda")
        say(f"[audit variant] {w.name} scale={scale}")
        y = run(inp, "tiled", tfl.AUDIT_LIB_PATH, counters)
        got = counters.cpu().numpy()
        assert int(got[SLOTS["split_wg"]]) == want_split, (scale, got.tolist())
        assert int(got[SLOTS["bounded_wg"]]) == want_bounded, (scale, got.tolist())
        assert_gate(y, oracle_forward(inp), f"{w.name} scale {scale}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_pq_score_variant_follows_magnitude(dtype):
    """The PQ attention tasks pick their score variant as the layer-wise
    kernels do, from the row-norm maxima of their (sequence, head), formed
    for every layer: split only in the first layer and only where a single
    fp16 pass's score error bound exceeds 2^-8; bounded where every score is
    within +-14 in exp2 units.  Every layer has the same N attention tasks.
    Scale 1: no task splits, all 2N are bounded.  Scale 1e3: the N
    first-layer tasks split and are not bounded, the N second-layer tasks
    (LayerNorm-bounded input) are bounded.  The outputs meet the gate."""
    import torch

    import masked_attention_causal_amd as tfl
    from tests.gate import assert_gate, oracle_forward
    w = W(f"a_pq_adapt_{dtype}", 2, 128, 2, 512, 2, 900, dtype, 1, 900, 1.0)
    n_att = None
    for scale in (1.0, 1e3):
        inp = synth.make_inputs(w, 11, scale=scale)
        counters = torch.zeros(8, dtype=torch.int64, device="cuda")
        say(f"[audit variant] {w.name} scale={scale}")
        y = run(inp, "pq", tfl.AUDIT_LIB_PATH, counters)
        got = counters.cpu().numpy()
        split, bounded = int(got[SLOTS["split_wg"]]), int(got[SLOTS["bounded_wg"]])
        if scale == 1.0:
            assert split == 0 and bounded > 0 and bounded % 2 == 0, got.tolist()
            n_att = bounded // 2
        else:
            assert split == n_att and bounded == n_att, (n_att, got.tolist())
        assert_gate(y, oracle_forward(inp), f"{w.name} scale {scale}")
