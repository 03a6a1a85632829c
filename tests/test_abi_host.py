"""Host-side checks of the C ABI (no GPU needed: tfl_create and every
argument check run before any device call)."""
import ctypes
import os
import re

import pytest

import masked_attention_causal_amd as tfl
from masked_attention_causal_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return tfl.load_library()


def declared_symbols():
    with open(os.path.join(ROOT, "include", "tfl.h")) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"\b(tfl_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_symbols()
    assert set(names) == set(tfl.SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_workload_plans():
    for name, w in synth.WORKLOADS.items():
        plan, path, ws = tfl.plan_for(w.n_layers, w.d, w.H, w.f, w.B, w.L, w.dtype)
        assert path in ("seq", "pq", "tiled"), (name, plan)
        assert ws > 0 or path == "seq"
        assert plan.upper().startswith(path.upper())


def test_dispatcher_rules():
    # short fp16/bf16 sequences stay on chip; fp32 I/O, long sequences and d > 256 go tiled
    assert tfl.plan_for(2, 256, 4, 1024, 4096, 64, "f16")[1] == "seq"
    assert tfl.plan_for(2, 256, 4, 1024, 7, 33, "bf16")[1] == "seq"
    assert tfl.plan_for(2, 256, 4, 1024, 4096, 65, "f16")[1] == "tiled"
    assert tfl.plan_for(2, 256, 4, 1024, 4096, 64, "f32")[1] == "tiled"
    assert tfl.plan_for(4, 1024, 16, 4096, 8, 512, "bf16")[1] == "tiled"
    assert tfl.plan_for(2, 64, 4, 256, 1, 100000, "f16")[1] == "tiled"
    with pytest.raises(tfl.TflError) as e:
        tfl.plan_for(2, 256, 4, 1024, 4, 128, "f16", force_path="seq")
    assert e.value.status == 2
    # tiny widths (d <= 64, L <= 64): the small sequence-resident kernel, any dtype
    assert tfl.plan_for(2, 32, 2, 128, 4, 32, "f32") == ("SEQ/small/1seq/f32", "seq", 0)
    assert tfl.plan_for(2, 64, 4, 256, 4, 32, "f32", force_path="seq")[1] == "seq"
    assert tfl.plan_for(2, 32, 2, 128, 4, 65, "f32")[1] == "tiled"
    with pytest.raises(tfl.TflError):
        tfl.plan_for(2, 128, 2, 512, 4, 64, "f32", force_path="seq")


def test_pq_dispatch_rules():
    # fewer (sequence, head, 64-query tile) units than compute units and no
    # sequence-resident fit -> PQ path (task list over 64-row tiles)
    assert tfl.plan_for(2, 128, 2, 512, 1, 4096, "f32")[1] == "pq"
    assert tfl.plan_for(2, 256, 4, 1024, 1, 1000, "bf16")[1] == "pq"
    assert tfl.plan_for(2, 128, 2, 512, 2, 4096, "f32")[1] == "tiled"    # 256 units
    assert tfl.plan_for(2, 128, 2, 96 * 5, 1, 4096, "f16")[1] == "tiled"  # FFN width not a multiple of 128
    assert tfl.plan_for(2, 64, 4, 256, 1, 4096, "f16")[1] == "tiled"      # head dim 16
    with pytest.raises(tfl.TflError) as e:
        tfl.plan_for(2, 64, 4, 256, 1, 300, "f16", force_path="pq")
    assert e.value.status == 2


def test_noalloc_refuses_plans_beyond_the_static_workspace(lib):
    # the d=1024 workload's layer-wise plan needs 136 MiB of workspace; the
    # static array holds 32 MiB: refused before any device call
    w = synth.WORKLOADS["gemm_d1024_b8_l512"]
    cfg = tfl.make_config(w.n_layers, w.d, w.H, w.f, w.B, w.L, w.dtype)
    h = tfl.Handle(cfg, [{k: 0x10000 for k in tfl.LAYER_KEYS}] * w.n_layers)
    assert h.workspace_bytes > tfl.binding.STATIC_WORKSPACE_BYTES
    with pytest.raises(tfl.TflError) as e:
        h.forward_noalloc_raw(0x100000, 0x200000, 0x300000, 0)
    assert e.value.status == 3 and "static workspace" in str(e.value)
    h.close()
    assert lib.tfl_forward_noalloc(None, 0x100000, 0x200000, 0x300000, None) == 1


def test_pq_single_launch_is_refused():
    # the single persistent launch of the PQ tasks stays disabled until the
    # cause of its one unfinished GPU run is shown (include/tfl.h)
    with pytest.raises(tfl.TflError) as e:
        tfl.plan_for(2, 128, 2, 512, 1, 4096, "f32", force_path="pq_single")
    assert e.value.status == 2 and "persistent" in str(e.value)


def test_audit_build_exports_and_product_does_not(lib):
    # the audit entry point (include/tfl_audit.h) exists only in the test build
    assert not hasattr(lib, "tfl_audit_attach")
    audit = tfl.load_library(tfl.AUDIT_LIB_PATH)
    assert ctypes.cast(audit.tfl_audit_attach, ctypes.c_void_p).value
    for n in declared_symbols():
        assert hasattr(audit, n), n


def test_pq_workspace_layout():
    n_layers, d, H, f, B, L = 2, 128, 2, 512, 1, 4096
    plan, path, ws = tfl.plan_for(n_layers, d, H, f, B, L, "f32", force_path="pq")
    assert path == "pq" and plan.startswith("PQ/")
    up = lambda v: (v + 255) // 256 * 256
    NT = (L + 63) // 64
    ks = 8
    q, r = NT // ks, NT % ks
    pairs = NT + ks * q * (q - 1) // 2 + q * r          # (tile, split) pairs per (sequence, head)
    assert pairs == sum(t // ks + 1 for t in range(NT))
    T, dh, Lp = B * L, d // H, NT * 64
    weights = n_layers * (4 * d * d + 2 * d * f) * 2 * 2     # fp16 hi and lo planes of every GEMM weight
    fs = 4                                                  # FFN tasks per tile: 4 x 64 tiles fill 256 CUs
    need = (up(T * d * 4) + up(T * d * 4) + up(T * d * 4 * fs)   # residual, X1, FFN partials
            + 2 * up(T * d * 2 * n_layers) + 2 * up(T * d * 2)
            + up(B * d * Lp * 2 * n_layers) + up(B * H * pairs * 64 * dh * 2) + up(B * H * pairs * 64 * 8)
            + up(B * H * NT * 8)                                 # per (sequence, head, tile) Q/K norm bounds
            + up(weights))
    assert ws == need
    # fp16 I/O reads the given weights: no planes
    ws16 = tfl.plan_for(n_layers, d, H, f, B, L, "f16", force_path="pq")[2]
    assert ws16 == need - up(weights) - (up(T * d * 4) - up(T * d * 4))


def test_workspace_covers_the_tiled_buffers():
    # d_model <= 256, 16-bit I/O: fused row kernel, no Z / X1 / FFN buffers:
    # residual, Q, K (fp32-sized: hi and lo fp16 planes), A, O, V^T
    w = synth.WORKLOADS["stream_d64_b1_l100000"]
    plan, _, ws = tfl.plan_for(w.n_layers, w.d, w.H, w.f, w.B, w.L, w.dtype, force_path="tiled")
    assert plan.endswith("/rowfused"), plan
    T = w.B * w.L
    Lp = (w.L + 127) // 128 * 128          # V^T rows padded to whole 128-key tiles
    stats = w.B * w.H * -(-w.L // 256) * 8     # per-layer Q/K row-norm maxima per 256 rows
    need = 3 * T * w.d * 4 + 2 * T * w.d * 2 + w.B * w.d * Lp * 2 + stats
    assert need <= ws <= need + 7 * 256
    # d_model 1024, bf16 I/O: separate kernels, all buffers, plus every
    # layer's four GEMM weights converted to one fp16 plane
    w = synth.WORKLOADS["gemm_d1024_b8_l512"]
    plan, _, ws = tfl.plan_for(w.n_layers, w.d, w.H, w.f, w.B, w.L, w.dtype)
    assert not plan.endswith("/rowfused"), plan
    T = w.B * w.L
    Lp = (w.L + 127) // 128 * 128
    wts = w.n_layers * (4 * w.d * w.d + 2 * w.d * w.f)
    stats = w.B * w.H * -(-w.L // 256) * 8
    need = 5 * T * w.d * 4 + 2 * T * w.d * 2 + w.B * w.d * Lp * 2 + T * w.f * 2 + wts * 2 + stats
    assert need <= ws <= need + 11 * 256
    # fp32 I/O stays on the separate kernels, with two fp16 planes (hi, lo)
    # for every operand and weight
    L, d, f, n_layers = 4096, 64, 256, 2
    plan, _, ws = tfl.plan_for(n_layers, d, 4, f, 1, L, "f32", force_path="tiled")
    assert not plan.endswith("/rowfused") and "f16x3" in plan, plan
    need = 5 * L * d * 4 + 2 * L * d * 4 + d * L * 2 + L * f * 4 + n_layers * (4 * d * d + 2 * d * f) * 4
    assert need <= ws <= need + 10 * 256


@pytest.mark.parametrize("cfg,status", [
    (dict(n_layers=0), 1), (dict(d_model=0), 1), (dict(batch=0), 1), (dict(seq_len=-3), 1),
    (dict(n_heads=3), 1), (dict(dtype=7), 1), (dict(force_path=9), 1),
    (dict(d_model=48, n_heads=1), 2), (dict(d_model=256, n_heads=2), 2), (dict(d_ffn=100), 2),
    (dict(d_model=2048, n_heads=32), 2), (dict(batch=70000), 2),
    (dict(d_model=288, n_heads=9), 2), (dict(d_model=352, n_heads=11), 2), (dict(d_model=960, n_heads=15), 2),
])
def test_create_rejects(cfg, status):
    base = dict(n_layers=2, d_model=64, n_heads=4, d_ffn=128, batch=2, seq_len=16, dtype="f16")
    base.update(cfg)
    with pytest.raises(tfl.TflError) as e:
        tfl.plan_for(**base)
    assert e.value.status == status
    assert "tfl_create" in str(e.value)


def test_create_accepts_d_model_with_small_odd_part():
    # multiples of 32 up to 1024 whose odd part is at most 7 (the LayerNorm
    # row split); the others are rejected above
    for k in (1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16, 20, 24, 28, 32):
        d = 32 * k
        tfl.plan_for(1, d, d // 32, 2 * d, 2, 16, "f16", force_path="tiled")


def test_create_rejects_bad_layer_pointers(lib):
    cfg = tfl.make_config(1, 64, 4, 128, 2, 16, "f16")
    good = {k: 0x10000 for k in tfl.LAYER_KEYS}
    for key, val in (("w_qkv", 0), ("w_1", 0x10008), ("b_o", 0x10001), ("ln1_g", 0x10002), ("ln2_b", 0)):
        bad = dict(good)
        bad[key] = val
        with pytest.raises(tfl.TflError) as e:
            tfl.Handle(cfg, [bad])
        assert e.value.status == 1


def test_forward_argument_checks_before_any_device_call(lib):
    cfg = tfl.make_config(1, 64, 4, 128, 2, 16, "f16", force_path="tiled")   # a plan with a workspace
    h = tfl.Handle(cfg, [{k: 0x10000 for k in tfl.LAYER_KEYS}])
    n = h.workspace_bytes
    X, Y, LN, WS = 0x100000, 0x200000, 0x300000, 0x400000
    cases = [
        ((0, LN, Y, WS, n), 1),           # null x
        ((X, 0, Y, WS, n), 1),            # null lens
        ((X + 8, LN, Y, WS, n), 1),       # misaligned x
        ((X, LN, Y, WS, n - 1), 3),       # workspace too small
        ((X, LN, Y, WS + 16, n), 1),      # workspace misaligned
        ((X, LN, X + 256, WS, n), 1),     # y overlaps x
        ((X, LN, WS + 512, WS, n), 1),    # y overlaps workspace
        ((WS + 256, LN, Y, WS, n), 1),    # x overlaps workspace
    ]
    for args, status in cases:
        with pytest.raises(tfl.TflError) as e:
            h.forward_raw(*args, 0)
        assert e.value.status == status, args
    st = lib.tfl_forward(None, X, LN, Y, WS, n, None)
    assert st == 1
    h.close()


def test_null_handle_queries(lib):
    assert lib.tfl_plan_path(None) == -1
    assert lib.tfl_destroy(None) == 0
    n = ctypes.c_size_t()
    assert lib.tfl_workspace_bytes(None, ctypes.byref(n)) == 1


def test_library_does_not_link_the_oracle():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", tfl.LIB_PATH], capture_output=True, text=True).stdout
    assert "orc_" not in out
    src = os.path.join(ROOT, "masked_attention_causal_amd", "csrc")
    for f in os.listdir(src):
        if not os.path.isfile(os.path.join(src, f)):
            continue
        with open(os.path.join(src, f)) as fh:
            assert "oracle" not in fh.read().lower(), f
