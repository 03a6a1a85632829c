"""GPU parity of the PQ path (task list over 64-row tiles, one launch per
stage) against the fp64 oracle.

Shapes cover every (d, head dim) the path supports, the three I/O dtypes,
ragged sequence ends (L not a multiple of 64), several key splits per query
tile (L > 8 * 64), more than one sequence, one to three layers, lengths of 1
and of L, and the input scales 1e-3, 1 and 1e3 under the same gate as every
other path.
"""
import numpy as np
import pytest

from masked_attention_causal_amd import synth
from tests.gate import assert_gate, gpu_forward, oracle_forward, say

pytestmark = pytest.mark.gpu

W = synth.Workload

PQ_SHAPES = [
    W("q_f32_d128_dh64", 2, 128, 2, 512, 1, 1000, "f32", 900, 1000, 1.0),
    W("q_f16_d256_dh64", 2, 256, 4, 256, 2, 600, "f16", 1, 600, 1.0),
    W("q_bf16_d64_dh32", 3, 64, 2, 128, 2, 700, "bf16", 1, 700, 1.0),
    W("q_f32_d64_dh64", 1, 64, 1, 128, 1, 130, "f32", 1, 130, 1.0),
    W("q_f16_d128_dh32", 2, 128, 4, 384, 3, 333, "f16", 1, 333, 1.0),
    W("q_f32_d256_dh32", 2, 256, 8, 256, 1, 300, "f32", 1, 300, 1.0),
    W("q_bf16_d256_dh64", 1, 256, 4, 512, 1, 1100, "bf16", 1100, 1100, 1.0),
]


@pytest.mark.parametrize("w", PQ_SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("scale", [1e-3, 1.0, 1e3])
def test_pq_shapes(w, scale):
    import masked_attention_causal_amd as tfl
    plan, path, _ = tfl.plan_for(w.n_layers, w.d, w.H, w.f, w.B, w.L, w.dtype, force_path="pq")
    assert path == "pq"
    for seed in (0, 1):
        inp = synth.make_inputs(w, seed, scale=scale, affine=(seed == 1))
        inp.lens[0] = w.L
        if w.B > 1:
            inp.lens[1] = 1
        say(f"[pq] {w.name} plan={plan} seed={seed} scale={scale} lens={inp.lens.tolist()}")
        assert_gate(gpu_forward(inp, force_path="pq"), oracle_forward(inp), f"{w.name} seed {seed} scale {scale}")


INV = W("inv_pq", 2, 128, 2, 256, 3, 700, "f16", 1, 700, 1.0)


def test_pq_invariances_bit_exact():
    inp = synth.make_inputs(INV, 4, lens=np.array([700, 300, 5], np.int32))
    y = gpu_forward(inp, force_path="pq")
    p = synth.make_inputs(INV, 4, lens=inp.lens)
    p.x = inp.x.copy()
    p.x[1, 500] = synth.round_to(synth.to_f64(p.x[1, 500], "f16") + 1.0, "f16")    # padding position
    p.x[0, 600] = synth.round_to(synth.to_f64(p.x[0, 600], "f16") - 1.0, "f16")    # causal position
    say("[pq invariance] perturbed padding and causal positions")
    y2 = gpu_forward(p, force_path="pq")
    assert np.array_equal(y[0, :600], y2[0, :600])
    assert not np.array_equal(y[0, 600:], y2[0, 600:])
    keep = np.ones(INV.L, bool)
    keep[500] = False
    assert np.array_equal(y[1, keep], y2[1, keep])
    assert np.array_equal(y[2], y2[2])
    say("[pq determinism]")
    assert np.array_equal(y, gpu_forward(inp, force_path="pq"))
    for b in range(INV.B):
        say(f"[pq batch independence] sequence {b} alone")
        assert np.array_equal(gpu_forward(synth.subset(inp, [b]), force_path="pq")[0], y[b])


def test_pq_check_mode_and_clamped_lengths(monkeypatch):
    import torch

    import masked_attention_causal_amd as tfl
    w = W("err_pq", 1, 64, 2, 128, 2, 80, "f16", 1, 80, 1.0)
    inp = synth.make_inputs(w, 0)
    layers = [{k: tfl.to_device(v, w.dtype) for k, v in lw.items()} for lw in inp.layers]
    enc = tfl.Encoder(w.n_layers, w.d, w.H, w.f, w.B, w.L, w.dtype, layers, force_path="pq")
    assert enc.plan_path == "pq"
    x = tfl.to_device(inp.x, w.dtype)
    lens = torch.from_numpy(inp.lens).cuda()
    y = torch.empty_like(x)
    h = enc.handle
    ws = enc.workspace()
    st = torch.cuda.current_stream().cuda_stream
    with pytest.raises(tfl.TflError) as e:
        h.forward_raw(x.data_ptr(), lens.data_ptr(), y.data_ptr(), ws.data_ptr(), h.workspace_bytes - 1, st)
    assert e.value.status == 3
    bad = torch.tensor([0, 81], dtype=torch.int32, device="cuda")
    monkeypatch.setenv("TFL_CHECK", "1")
    with pytest.raises(tfl.TflError) as e:
        h.forward_raw(x.data_ptr(), bad.data_ptr(), y.data_ptr(), ws.data_ptr(), h.workspace_bytes, st)
    assert e.value.status == 1
    # a good forward passes the host-side length check
    h.forward_raw(x.data_ptr(), lens.data_ptr(), y.data_ptr(), ws.data_ptr(), h.workspace_bytes, st)
    monkeypatch.delenv("TFL_CHECK")
    say("[pq clamp] lengths 0 and 81 behave as 1 and L")
    h.forward_raw(x.data_ptr(), bad.data_ptr(), y.data_ptr(), ws.data_ptr(), h.workspace_bytes, st)
    torch.cuda.synchronize()
    clamped = synth.make_inputs(w, 0, lens=np.array([1, 80], np.int32))
    assert_gate(tfl.to_numpy_f64(y), oracle_forward(clamped), "pq clamped lengths")
    enc.close()


def test_pq_repeated_forwards_reuse_the_workspace():
    # every forward overwrites the partial attention states it reads: back-to-
    # back calls on one workspace give identical results
    import torch

    import masked_attention_causal_amd as tfl
    w = W("rep_pq", 2, 128, 2, 256, 1, 900, "f32", 900, 900, 1.0)
    inp = synth.make_inputs(w, 2)
    layers = [{k: tfl.to_device(v, w.dtype) for k, v in lw.items()} for lw in inp.layers]
    enc = tfl.Encoder(w.n_layers, w.d, w.H, w.f, w.B, w.L, w.dtype, layers, force_path="pq")
    x = tfl.to_device(inp.x, w.dtype)
    lens = torch.from_numpy(inp.lens).cuda()
    ws = enc.workspace()
    outs = []
    for i in range(4):
        y = torch.empty_like(x)
        enc.forward(x, lens, y, ws)
        outs.append(y)
    torch.cuda.synchronize()
    ys = [tfl.to_numpy_f64(o) for o in outs]
    for i in range(1, 4):
        assert np.array_equal(ys[0], ys[i]), i
    assert_gate(ys[0], oracle_forward(inp), "pq repeated")
    enc.close()


@pytest.mark.skip(reason="the single persistent launch of the PQ tasks (TFL_PATH_PQ_SINGLE) is disabled: "
                         "its one GPU run did not finish and no cause has been shown; tfl_create returns "
                         "TFL_E_UNSUPPORTED for it (checked on the CPU in tests/test_abi_host.py)")
@pytest.mark.parametrize("scale", [1e-3, 1.0, 1e3])
def test_pq_single_launch(scale):
    w = synth.WORKLOADS["latency_d128_b1_l4096"]
    inp = synth.make_inputs(w, 0, scale)
    say(f"[pq single] scale={scale}")
    assert_gate(gpu_forward(inp, force_path="pq_single"), oracle_forward(inp), f"pq single scale {scale}")
