"""Pins of the FP8 oracle: the E4M3 code table against its closed form,
rounding against torch's float8_e4m3fn conversion and hand-derived ties,
exactness on inputs already on the grid, the error bound of per-tensor
quantisation, and the structure of the FP8 decoder layer."""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as Q
from oracle import ModelDims, LayerWeights


def test_code_table_closed_form():
    v = Q.e4m3_values()
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x77] == 240.0 and v[0xB8] == -1.0
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x07] == 7 * 2.0 ** -9
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.sum(np.isfinite(v)) == 254
    assert np.all(np.diff(v[:0x7F]) > 0)


def test_code_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = Q.e4m3_values()
    fin = np.isfinite(v)
    assert np.array_equal(v[fin], codes[fin]) and np.all(np.isnan(codes[~fin]))


def test_rounding_matches_torch_and_hand_ties():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 0.01, 20000),
                        rng.normal(0, 1, 20000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(Q.round_e4m3(x), ref)
    # ties to the even mantissa, by hand: 1 + 1/16 between 1 and 1.125; 1.1875 between
    # 1.125 and 1.25; 248 between 240 and 256; 3 * 2^-10 between the subnormals 2^-9 and 2^-8
    np.testing.assert_array_equal(Q.round_e4m3([1.0625, 1.1875, 248.0, 3 * 2.0 ** -10, 2.0 ** -10]),
                                  [1.0, 1.25, 256.0, 2.0 ** -8, 0.0])
    with pytest.raises(ValueError):
        Q.round_e4m3([449.0])


def test_quantize_scale_and_error_bound():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(64, 96)) * 3
    q, s = Q.quantize(x)
    amax = np.max(np.abs(x.astype(np.float32)))
    assert s == pytest.approx(amax / 448, rel=1e-7)
    assert np.max(np.abs(q)) == 448.0                         # the largest element maps to 448
    # relative error of normal-range values at most half an ulp (2^-4) plus the fp32 step
    big = np.abs(x) > 2.0 ** -6 * s
    assert np.max(np.abs(q * s - x)[big] / np.abs(x)[big]) <= 2.0 ** -4 * (1 + 1e-6)
    q0, s0 = Q.quantize(np.zeros((3, 4)))
    assert np.all(q0 == 0)


def test_linear_exact_on_grid_values():
    # integers up to 16 are E4M3 values; with amax 448 the factor is 1 and nothing rounds
    rng = np.random.default_rng(2)
    x = rng.integers(-16, 17, size=(8, 32)).astype(np.float64)
    x[0, 0] = 448
    w = rng.integers(-16, 17, size=(12, 32)).astype(np.float64)
    w[0, 0] = -448
    qw, sw = Q.quantize(w)
    assert sw == 1.0
    np.testing.assert_array_equal(Q.linear_fp8(x, qw, sw), x @ w.T)


def test_fp8_layer_structure():
    rng = np.random.default_rng(3)
    d = ModelDims(hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, intermediate=96,
                  rms_eps=1e-6, rope_theta=1e4, mrope_section=(3, 3, 2))
    S = 12
    g = lambda *sh: rng.normal(size=sh) * 0.1
    w = LayerWeights(ln_in=rng.uniform(0.5, 1.5, 64), w_q=g(64, 64), w_k=g(32, 64), w_v=g(32, 64),
                     q_norm=rng.uniform(0.5, 1.5, 16), k_norm=rng.uniform(0.5, 1.5, 16),
                     w_o=g(64, 64), ln_post=rng.uniform(0.5, 1.5, 64), w_gate=g(96, 64),
                     w_up=g(96, 64), w_down=g(64, 96))
    h = rng.normal(size=(S, 64))
    pos = np.tile(np.arange(S), (3, 1))
    cos, sin = oracle.rope_cos_sin(pos, 16, 1e4, (3, 3, 2))
    ref = oracle.decoder_layer(h, w, cos, sin, d)
    got = Q.decoder_layer_fp8(h, w, Q.quantize_layer(w), cos, sin, d)
    delta = got - h
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref - h)
    assert 1e-3 < rel < 0.1          # the layer's update carries FP8-sized errors, no more
    # zero output projections: the layer is the identity, exactly
    w0 = LayerWeights(**{**w.__dict__, "w_o": np.zeros((64, 64)), "w_down": np.zeros((64, 96))})
    np.testing.assert_array_equal(Q.decoder_layer_fp8(h, w0, Q.quantize_layer(w0), cos, sin, d), h)


def _layer(rng):
    d = ModelDims(hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, intermediate=96,
                  rms_eps=1e-6, rope_theta=1e4, mrope_section=(3, 3, 2))
    g = lambda *sh: rng.normal(size=sh) * 0.1
    w = LayerWeights(ln_in=rng.uniform(0.5, 1.5, 64), w_q=g(64, 64), w_k=g(32, 64), w_v=g(32, 64),
                     q_norm=rng.uniform(0.5, 1.5, 16), k_norm=rng.uniform(0.5, 1.5, 16),
                     w_o=g(64, 64), ln_post=rng.uniform(0.5, 1.5, 64), w_gate=g(96, 64),
                     w_up=g(96, 64), w_down=g(64, 96))
    return d, w


def test_fp8_layer_scale_bookkeeping_is_equivariant():
    # Scaling a weight by a power of two leaves its FP8 codes alone and scales its
    # per-tensor scale: the contribution of the o projection (with the MLP switched off)
    # and of the down projection must scale by the same factor, to fp64 rounding (a scale
    # taken from the wrong tensor breaks this).
    rng = np.random.default_rng(4)
    d, w = _layer(rng)
    S = 10
    h = rng.normal(size=(S, 64))
    cos, sin = oracle.rope_cos_sin(np.tile(np.arange(S), (3, 1)), 16, 1e4, (3, 3, 2))
    run = lambda ww: Q.decoder_layer_fp8(h, ww, Q.quantize_layer(ww), cos, sin, d)
    w_nomlp = LayerWeights(**{**w.__dict__, "w_down": np.zeros((64, 96))})
    attn = run(w_nomlp) - h
    w4 = LayerWeights(**{**w_nomlp.__dict__, "w_o": w.w_o * 4.0})
    np.testing.assert_allclose(run(w4) - h, 4.0 * attn, rtol=1e-9, atol=1e-12)
    base = run(w_nomlp)
    mlp = run(w) - base
    w4 = LayerWeights(**{**w.__dict__, "w_down": w.w_down * 4.0})
    np.testing.assert_allclose(run(w4) - base, 4.0 * mlp, rtol=1e-9, atol=1e-12)


def test_fused_linears_share_one_scale():
    # Weights on the E4M3 grid whose fused tensor has max |w| = 448 quantise with scale 1
    # and no rounding: every dequantised weight equals the original, in every part of the
    # fused qkv and gate_up tensors. Parts quantised on their own would have smaller
    # maxima (16 here), factors of 28 and rounded codes (3 * 28 = 84 is a tie between 80
    # and 88).
    rng = np.random.default_rng(5)
    d, w = _layer(rng)
    ints = lambda a: rng.integers(-16, 17, size=a.shape).astype(np.float64)
    parts = {k: ints(getattr(w, k)) for k in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")}
    parts["w_q"][0, 0] = 448.0
    parts["w_gate"][0, 0] = -448.0
    parts["w_o"][0, 0] = 448.0
    parts["w_down"][0, 0] = 448.0
    parts["w_k"][0, 0] = parts["w_up"][0, 0] = 3.0
    wg = LayerWeights(**{**w.__dict__, **parts})
    qw = Q.quantize_layer(wg)
    for name, stacked in (("w_qkv", ("w_q", "w_k", "w_v")), ("w_gate_up", ("w_gate", "w_up")),
                          ("w_o", ("w_o",)), ("w_down", ("w_down",))):
        vals, s = qw[name]
        assert s == 1.0
        np.testing.assert_array_equal(vals, np.concatenate([parts[p] for p in stacked]))


def test_threaded_quantisation_is_the_same_function():
    """quantize(x, threads) forms the codes of row blocks concurrently: the
    values and the scale equal the one-pass result bit for bit (ragged block
    edges, an all-zero tensor and a tensor too short to split included)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1037, 96)) * np.exp2(rng.integers(-12, 4, size=(1037, 1)))
    for t in (2, 7):
        q1, s1 = Q.quantize(x)
        qt, st = Q.quantize(x, threads=t)
        assert st == s1 and np.array_equal(q1, qt)
    z, sz = Q.quantize(np.zeros((50, 8)), threads=4)
    assert sz == 1.0 and not z.any()
    q1, _ = Q.quantize(x[:5])
    qt, _ = Q.quantize(x[:5], threads=4)
    assert np.array_equal(q1, qt)
