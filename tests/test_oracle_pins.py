"""Pins of the fp64 CPU oracle against things other than itself.

Each test fixes one part of the oracle to an independent statement of what it
must compute: a library implementation (PyTorch's encoder layer, SDPA,
layer_norm; mpmath's erf), brute force on tiny inputs, a closed form, or an
invariant of the mathematics.  A dropped term, a wrong sign or index or a
transposed operand in ``oracle/oracle.c`` fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from masked_attention_causal_amd import synth

RNG = np.random.default_rng(1234)


def rand_layers(n_layers, d, f, rng, affine=True):
    out = []
    for _ in range(n_layers):
        lw = {
            "w_qkv": rng.standard_normal((3 * d, d)) * 0.3,
            "w_o": rng.standard_normal((d, d)) * 0.3,
            "w_1": rng.standard_normal((f, d)) * 0.3,
            "w_2": rng.standard_normal((d, f)) * 0.3,
            "b_qkv": rng.standard_normal(3 * d) * (0.2 if affine else 0),
            "b_o": rng.standard_normal(d) * (0.2 if affine else 0),
            "b_1": rng.standard_normal(f) * (0.2 if affine else 0),
            "b_2": rng.standard_normal(d) * (0.2 if affine else 0),
            "ln1_g": 1 + rng.standard_normal(d) * (0.3 if affine else 0),
            "ln1_b": rng.standard_normal(d) * (0.3 if affine else 0),
            "ln2_g": 1 + rng.standard_normal(d) * (0.3 if affine else 0),
            "ln2_b": rng.standard_normal(d) * (0.3 if affine else 0),
        }
        out.append(lw)
    return out


def torch_stack(x, lens, layers, H, eps=1e-5):
    """PyTorch's own post-LN encoder layer, float64, dropout 0, exact GELU,
    bool causal mask plus key-padding mask, applied layer by layer."""
    B, L, d = x.shape
    f = layers[0]["w_1"].shape[0]
    t = torch.from_numpy(x)
    causal = torch.triu(torch.ones(L, L, dtype=torch.bool), 1)          # True = masked
    pad = torch.arange(L)[None, :] >= torch.from_numpy(np.asarray(lens))[:, None].long()
    for lw in layers:
        m = torch.nn.TransformerEncoderLayer(d, H, f, dropout=0.0, activation="gelu",
                                             layer_norm_eps=eps, batch_first=True,
                                             norm_first=False, dtype=torch.float64)
        m.train()  # the plain (non-fused) path; dropout is 0 so this is deterministic
        sd = {
            "self_attn.in_proj_weight": lw["w_qkv"], "self_attn.in_proj_bias": lw["b_qkv"],
            "self_attn.out_proj.weight": lw["w_o"], "self_attn.out_proj.bias": lw["b_o"],
            "linear1.weight": lw["w_1"], "linear1.bias": lw["b_1"],
            "linear2.weight": lw["w_2"], "linear2.bias": lw["b_2"],
            "norm1.weight": lw["ln1_g"], "norm1.bias": lw["ln1_b"],
            "norm2.weight": lw["ln2_g"], "norm2.bias": lw["ln2_b"],
        }
        m.load_state_dict({k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in sd.items()})
        with torch.no_grad():
            t = m(t, src_mask=causal, src_key_padding_mask=pad)
    return t.numpy()


# ---------------------------------------------------------------- whole layer


@pytest.mark.parametrize("B,L,d,H,f,nl", [(3, 9, 12, 3, 20, 2), (2, 17, 16, 2, 40, 3), (1, 5, 8, 1, 8, 1)])
def test_stack_matches_torch_encoder_layer(orc, B, L, d, H, f, nl):
    """Library pin: nn.TransformerEncoderLayer (post-LN, GELU, both masks)."""
    rng = np.random.default_rng(B * 100 + L)
    x = rng.standard_normal((B, L, d))
    lens = rng.integers(1, L + 1, size=B).astype(np.int32)
    lens[0] = L
    if B > 1:
        lens[1] = 1
    layers = rand_layers(nl, d, f, rng)
    y = orc.forward(x, lens, layers, H)
    ref = torch_stack(x, lens, layers, H)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-11)


def test_stack_matches_torch_at_extreme_scales(orc):
    """Same pin at input scales 1e-3 and 1e3 (near-tied and peaked softmax)."""
    rng = np.random.default_rng(7)
    B, L, d, H, f = 2, 12, 16, 4, 32
    layers = rand_layers(2, d, f, rng, affine=False)
    lens = np.array([12, 7], np.int32)
    for s in (1e-3, 1e3):
        x = rng.standard_normal((B, L, d)) * s
        np.testing.assert_allclose(orc.forward(x, lens, layers, H), torch_stack(x, lens, layers, H),
                                   rtol=1e-9, atol=1e-10)


def test_ln_eps_is_used(orc):
    """eps enters as sqrt(var + eps): at input scale 1e-3 it changes the output."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 6, 8)) * 1e-3
    layers = rand_layers(1, 8, 16, rng, affine=False)
    lens = np.array([6], np.int32)
    a = orc.forward(x, lens, layers, 2, eps=1e-5)
    b = orc.forward(x, lens, layers, 2, eps=1e-12)
    assert np.abs(a - b).max() > 1e-3
    np.testing.assert_allclose(b, torch_stack(x, lens, layers, 2, eps=1e-12), rtol=1e-9, atol=1e-9)


# ---------------------------------------------------------------- attention


def dense_masked_attention(qkv, lens, H):
    """Brute force: explicit L x L boolean mask, -inf fill, dense softmax."""
    B, L, d3 = qkv.shape
    d = d3 // 3
    dh = d // H
    out = np.zeros((B, L, d))
    for b in range(B):
        ii, jj = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
        allowed = (jj <= ii) & (jj < lens[b])
        for h in range(H):
            q = qkv[b, :, h * dh:(h + 1) * dh]
            k = qkv[b, :, d + h * dh:d + (h + 1) * dh]
            v = qkv[b, :, 2 * d + h * dh:2 * d + (h + 1) * dh]
            s = q @ k.T / math.sqrt(dh)
            s = np.where(allowed, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[b, :, h * dh:(h + 1) * dh] = p @ v
    return out


@pytest.mark.parametrize("L", [1, 2, 5, 16])
def test_attention_brute_force_every_length(orc, L):
    H, d = 2, 8
    lens = np.arange(1, L + 1, dtype=np.int32)          # every valid length
    rng = np.random.default_rng(L)
    qkv = rng.standard_normal((L, L, 3 * d)) * 2.0
    o = orc.attention(qkv, lens, H)
    np.testing.assert_allclose(o, dense_masked_attention(qkv, lens, H), rtol=1e-13, atol=1e-14)


def test_attention_matches_sdpa(orc):
    """Library pin: F.scaled_dot_product_attention in float64 with a bool mask."""
    B, L, H, dh = 3, 23, 4, 8
    d = H * dh
    rng = np.random.default_rng(11)
    qkv = rng.standard_normal((B, L, 3 * d))
    lens = np.array([23, 1, 9], np.int32)
    o = orc.attention(qkv, lens, H)
    t = torch.from_numpy(qkv).view(B, L, 3, H, dh).permute(2, 0, 3, 1, 4)
    i = torch.arange(L)
    allowed = (i[None, :] <= i[:, None])[None] & (i[None, None, :] < torch.from_numpy(lens).long()[:, None, None])
    ref = torch.nn.functional.scaled_dot_product_attention(t[0], t[1], t[2], attn_mask=allowed[:, None])
    ref = ref.permute(0, 2, 1, 3).reshape(B, L, d).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_attention_single_key_returns_v0(orc):
    """Closed form: len_b = 1 leaves key 0 alone, so every row is exactly v_0."""
    B, L, H, d = 2, 7, 2, 8
    rng = np.random.default_rng(5)
    qkv = rng.standard_normal((B, L, 3 * d)) * 10
    o = orc.attention(qkv, np.array([1, 1], np.int32), H)
    for b in range(B):
        assert np.array_equal(o[b], np.broadcast_to(qkv[b, 0, 2 * d:], (L, d)))


def test_attention_zero_scores_is_prefix_mean(orc):
    """Closed form: q = k = 0 makes the softmax uniform over allowed keys."""
    B, L, H, d = 2, 9, 3, 6
    rng = np.random.default_rng(6)
    qkv = rng.standard_normal((B, L, 3 * d))
    qkv[:, :, :2 * d] = 0.0
    lens = np.array([9, 4], np.int32)
    o = orc.attention(qkv, lens, H)
    for b in range(B):
        for i in range(L):
            n = min(i, lens[b] - 1) + 1
            np.testing.assert_allclose(o[b, i], qkv[b, :n, 2 * d:].mean(axis=0), rtol=1e-14, atol=1e-15)


def test_attention_peaked_picks_argmax(orc):
    """Closed form: with a score gap above 50 the output is v at the argmax."""
    L, H, d = 8, 1, 4
    qkv = np.zeros((1, L, 3 * d))
    rng = np.random.default_rng(8)
    qkv[0, :, 2 * d:] = rng.standard_normal((L, d))
    qkv[0, :, 0] = 1.0                                  # q = e_0
    qkv[0, :, d] = np.arange(L) * 200.0                 # key j scores 100 j (dh = 4)
    o = orc.attention(qkv, np.array([5], np.int32), H)
    for i in range(L):
        j = min(i, 4)                                   # latest allowed key wins
        np.testing.assert_allclose(o[0, i], qkv[0, j, 2 * d:], rtol=1e-15, atol=1e-20 + np.exp(-50.0))


def test_attention_masked_keys_contribute_nothing(orc):
    """Invariant: keys j > i or j >= len_b never change the output."""
    B, L, H, d = 2, 10, 2, 8
    rng = np.random.default_rng(9)
    qkv = rng.standard_normal((B, L, 3 * d))
    lens = np.array([6, 10], np.int32)
    o = orc.attention(qkv, lens, H)
    q2 = qkv.copy()
    q2[0, 6:, d:] = rng.standard_normal((4, 2 * d)) * 100      # padded keys / values
    o2 = orc.attention(q2, lens, H)
    assert np.array_equal(o[1], o2[1])
    assert np.array_equal(o[0], o2[0])       # even padded query rows read keys < 6 only
    q3 = qkv.copy()
    q3[1, 7, d:] += 50.0                     # a future key for rows < 7
    o3 = orc.attention(q3, lens, H)
    assert np.array_equal(o[1, :7], o3[1, :7])
    assert not np.array_equal(o[1, 7:], o3[1, 7:])


def test_attention_rejects_bad_lengths(orc):
    qkv = np.zeros((1, 4, 6))
    for bad in (0, 5, -1):
        with pytest.raises(ValueError):
            orc.attention(qkv, np.array([bad], np.int32), 1)


# ---------------------------------------------------------------- LayerNorm


def test_layernorm_matches_torch(orc):
    rng = np.random.default_rng(10)
    z = rng.standard_normal((37, 24)) * 3 + 1
    g = rng.standard_normal(24)
    b = rng.standard_normal(24)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(z), (24,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    np.testing.assert_allclose(orc.layernorm(z, g, b, 1e-5), ref, rtol=1e-13, atol=1e-14)


def test_layernorm_constant_row_gives_beta(orc):
    z = np.full((3, 12), 0.1) * np.array([[1.0], [-7.0], [1e3]])
    g = np.linspace(0.5, 2, 12)
    b = np.linspace(-1, 1, 12)
    np.testing.assert_allclose(orc.layernorm(z, g, b, 1e-5), np.broadcast_to(b, z.shape), atol=1e-9)


def test_layernorm_moments(orc):
    """Before the affine map the row mean is 0 and the variance is
    var / (var + eps) (exactly 1 only when eps -> 0)."""
    rng = np.random.default_rng(12)
    for scale in (1e-3, 1.0, 1e3):
        z = rng.standard_normal((5, 64)) * scale + 0.5 * scale
        y = orc.layernorm(z, np.ones(64), np.zeros(64), 1e-5)
        var = z.var(axis=1)
        np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
        np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)


# ---------------------------------------------------------------- GELU


def test_gelu_matches_mpmath_erf(orc):
    import mpmath
    mpmath.mp.dps = 50
    xs = np.concatenate([np.linspace(-8, 8, 641), [-1e-3, 1e-3, -1e-8, 0.0, 3.3e-5]])
    g = orc.gelu(xs)
    for x, v in zip(xs, g):
        mx = mpmath.mpf(float(x))
        ref = mx / 2 * (1 + mpmath.erf(mx / mpmath.sqrt(2)))
        assert abs(v - float(ref)) <= 4e-16 * max(1.0, abs(x)), (x, v, float(ref))


def test_gelu_identities(orc):
    xs = np.linspace(-6, 6, 1201)
    g, gm = orc.gelu(xs), orc.gelu(-xs)
    np.testing.assert_allclose(g - gm, xs, atol=2e-15)
    assert orc.gelu(np.array([0.0]))[0] == 0.0


def test_gelu_is_not_polynomial_erf(orc):
    """An Abramowitz-Stegun style erf (abs error ~1e-7) would show here."""
    import mpmath
    mpmath.mp.dps = 40
    xs = np.linspace(-3, 3, 301)
    err = max(abs(v - float(mpmath.mpf(float(x)) / 2 * (1 + mpmath.erf(mpmath.mpf(float(x)) / mpmath.sqrt(2)))))
              for x, v in zip(xs, orc.gelu(xs)))
    assert err < 1e-14


# ---------------------------------------------------------------- products


def test_linear_matches_numpy(orc):
    rng = np.random.default_rng(13)
    A = rng.standard_normal((3, 5, 17))
    W = rng.standard_normal((11, 17))
    b = rng.standard_normal(11)
    np.testing.assert_allclose(orc.linear(A, W, b), A @ W.T + b, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(orc.linear(A, W), A @ W.T, rtol=1e-13, atol=1e-13)


def test_stage_functions_compose_to_forward(orc):
    """The per-stage entry points chain to exactly the whole-stack result."""
    rng = np.random.default_rng(14)
    B, L, d, H, f = 2, 11, 12, 3, 24
    x = rng.standard_normal((B, L, d))
    lens = np.array([11, 5], np.int32)
    layers = rand_layers(2, d, f, rng)
    X = x
    for lw in layers:
        qkv = orc.linear(X, lw["w_qkv"], lw["b_qkv"])
        o = orc.attention(qkv, lens, H)
        X1 = orc.out_ln(X, o, lw["w_o"], lw["b_o"], lw["ln1_g"], lw["ln1_b"])
        X = orc.ffn_ln(X1, lw["w_1"], lw["b_1"], lw["w_2"], lw["b_2"], lw["ln2_g"], lw["ln2_b"])
    assert np.array_equal(X, orc.forward(x, lens, layers, H))


# ---------------------------------------------------------------- stack invariants


def _case(seed=20, B=3, L=13, d=16, H=4, f=32):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L, d))
    lens = np.array([13, 6, 1][:B], np.int32)
    return x, lens, rand_layers(2, d, f, rng), H


def test_padding_invariance_bit_exact(orc):
    """Perturbing a padded position j >= len_b changes no other row."""
    x, lens, layers, H = _case()
    y = orc.forward(x, lens, layers, H)
    x2 = x.copy()
    x2[1, 9] += 3.0                       # len_1 = 6, so position 9 is padding
    y2 = orc.forward(x2, lens, layers, H)
    mask = np.ones(y.shape[:2], bool)
    mask[1, 9] = False
    assert np.array_equal(y[mask], y2[mask])
    assert not np.array_equal(y[1, 9], y2[1, 9])


def test_causal_prefix_bit_exact(orc):
    """Perturbing position j leaves rows i < j unchanged; later rows move."""
    x, lens, layers, H = _case()
    y = orc.forward(x, lens, layers, H)
    x2 = x.copy()
    x2[0, 7] -= 2.0
    y2 = orc.forward(x2, lens, layers, H)
    assert np.array_equal(y[0, :7], y2[0, :7])
    assert not np.array_equal(y[0, 8:], y2[0, 8:])
    assert np.array_equal(y[1:], y2[1:])


def test_prefix_forward_equals_full_forward(orc):
    x, lens, layers, H = _case()
    y = orc.forward(x, lens, layers, H)
    n = 8
    yp = orc.forward(x[:, :n], np.minimum(lens, n), layers, H)
    assert np.array_equal(y[:, :n], yp)


def test_batch_independence_bit_exact(orc):
    x, lens, layers, H = _case()
    y = orc.forward(x, lens, layers, H)
    for b in range(x.shape[0]):
        assert np.array_equal(orc.forward(x[b:b + 1], lens[b:b + 1], layers, H)[0], y[b])


def test_thread_count_independence(orc):
    x, lens, layers, H = _case(B=3, L=40)
    n0 = orc.max_threads()
    try:
        orc.set_threads(1)
        y1 = orc.forward(x, lens, layers, H)
        orc.set_threads(max(2, n0))
        y8 = orc.forward(x, lens, layers, H)
    finally:
        orc.set_threads(n0)
    assert np.array_equal(y1, y8)


# ---------------------------------------------------------------- generator


def test_round_to_f16_and_bf16_match_torch():
    """Library pin on float32-representable values (torch rounds float64 via
    float32, so only there is it a single rounding), plus a nearest-value
    check on raw float64 values."""
    vals = np.concatenate([RNG.standard_normal(20000) * 10.0 ** RNG.uniform(-6, 4, 20000),
                           [0.0, -0.0, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 65504.0, 6.1e-5, 1e-7]])
    v32 = vals.astype(np.float32).astype(np.float64)
    h = synth.round_to(v32, "f16")
    assert np.array_equal(h.astype(np.float64), torch.from_numpy(v32).to(torch.float16).double().numpy())
    bf = synth.round_to(v32, "bf16")
    ref = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf, ref)
    assert np.array_equal(synth.to_f64(bf, "bf16"), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())
    # float64 inputs: the stored f16 value is a nearest one (ties aside)
    h64 = synth.round_to(vals, "f16")
    up = np.nextafter(h64, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h64, np.float16(-np.inf)).astype(np.float64)
    e = np.abs(h64.astype(np.float64) - vals)
    assert np.all(e <= np.abs(up - vals)) and np.all(e <= np.abs(dn - vals))


def test_generator_is_seeded_and_shaped():
    w = synth.WORKLOADS["tiny_d32_b4_l32"]
    a = synth.make_inputs(w, 0)
    b = synth.make_inputs(w, 0)
    c = synth.make_inputs(w, 1)
    assert np.array_equal(a.x, b.x) and not np.array_equal(a.x, c.x)
    assert a.x.shape == (4, 32, 32) and a.x.dtype == np.float32
    assert a.lens.min() >= 1 and a.lens.max() <= 32
    assert len(a.layers) == 2 and a.layers[0]["w_qkv"].shape == (96, 32)
    big = synth.WORKLOADS["batch4096_d256_l64"]
    s = synth.make_inputs(big.with_batch(16), 0)
    assert 1e-3 <= s.scale <= 1e3 and s.x.dtype == np.float16
    assert s.lens.min() >= 8
