"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against what the pages and the mathematics fix:
hand-derived worked examples (``tests/golden``), closed forms, invariants,
special cases and independent library routines (torch's ``rms_norm``,
``scaled_dot_product_attention``, ``silu``; complex-number rotation). A
plausible slip in the oracle (a dropped eps, a wrong sign in rotate-half, a
``h % Hkv`` head map, a swapped gain, a transposed weight, DeepStack after the
wrong layer) fails at least one of them.
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import ModelDims, LayerWeights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def _vec(s):
    return np.array([float(x) for x in s.split(",")])


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_worked_examples():
    for ln in _lines("rmsnorm_worked.txt"):
        x, g, eps, y = [p.strip() for p in ln.split("|")]
        got = oracle.rms_norm(_vec(x)[None, :], _vec(g), float(eps))[0]
        np.testing.assert_allclose(got, _vec(y), rtol=1e-14, atol=1e-14)


def test_rmsnorm_unit_gain_output_rms():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(7, 96)) * rng.uniform(0.01, 10, size=(7, 1))
    eps = 1e-2
    y = oracle.rms_norm(x, np.ones(96), eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-12)


def test_rmsnorm_scale_invariant_without_eps():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(5, 64))
    g = rng.uniform(0.5, 1.5, size=64)
    np.testing.assert_allclose(oracle.rms_norm(37.0 * x, g, 0.0), oracle.rms_norm(x, g, 0.0), rtol=1e-12)


def test_rmsnorm_matches_torch_library():
    rng = np.random.default_rng(2)
    x = rng.normal(size=(9, 128))
    g = rng.uniform(0.5, 1.5, size=128)
    ref = F.rms_norm(torch.from_numpy(x), (128,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, g, 1e-6), ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- rotary

def _slot_fixture(name):
    table = {}
    for ln in _lines(name):
        axis, idx = ln.split(":")
        table[axis.strip()] = [int(v) for v in idx.split()]
    return table


@pytest.mark.parametrize("name,half,section", [("mrope_slots_d128.txt", 64, (24, 20, 20)),
                                               ("mrope_slots_d64.txt", 32, (24, 20, 20)),
                                               ("mrope_slots_d16_s221.txt", 8, (2, 2, 1))])
def test_mrope_slot_table(name, half, section):
    table = _slot_fixture(name)
    axes = oracle.mrope_slot_axes(half, section)
    for code, key in enumerate("THW"):
        assert sorted(np.flatnonzero(axes == code).tolist()) == table[key]


def test_rope_worked_example():
    kv = {}
    for ln in _lines("rope_worked.txt"):
        k, v = ln.split(":")
        kv[k.strip()] = [float(x) for x in v.split()]
    D = int(kv["head_dim"][0])
    theta = kv["theta"][0]
    section = [int(x) for x in kv["section"]]
    pos = np.array(kv["position"], dtype=np.int64).reshape(3, 1)
    angles = np.array(kv["angles"])
    cos, sin = oracle.rope_cos_sin(pos, D, theta, section)
    np.testing.assert_allclose(cos[0], np.cos(np.concatenate([angles, angles])), rtol=0, atol=1e-15)
    np.testing.assert_allclose(sin[0], np.sin(np.concatenate([angles, angles])), rtol=0, atol=1e-15)
    e0 = np.zeros((1, 1, D)); e0[0, 0, 0] = 1.0
    e4 = np.zeros((1, 1, D)); e4[0, 0, 4] = 1.0
    y0 = oracle.apply_rope(e0, cos, sin)[0, 0]
    y4 = oracle.apply_rope(e4, cos, sin)[0, 0]
    exp0 = np.zeros(D); exp0[0] = math.cos(5.0); exp0[4] = math.sin(5.0)
    exp4 = np.zeros(D); exp4[0] = -math.sin(5.0); exp4[4] = math.cos(5.0)
    np.testing.assert_allclose(y0, exp0, atol=1e-15)
    np.testing.assert_allclose(y4, exp4, atol=1e-15)


def test_rope_preserves_head_norm():
    rng = np.random.default_rng(3)
    S, Hh, D = 11, 3, 128
    x = rng.normal(size=(S, Hh, D))
    pos = rng.integers(0, 20000, size=(3, S))
    cos, sin = oracle.rope_cos_sin(pos, D, 5e6, (24, 20, 20))
    y = oracle.apply_rope(x, cos, sin)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)


def test_rope_equal_axes_is_textbook_complex_rotation():
    """All three axes equal -> 1-D RoPE: pair (d, d+D/2) rotated as x_d + i x_{d+D/2}."""
    rng = np.random.default_rng(4)
    S, Hh, D, theta = 13, 2, 64, 1e6
    x = rng.normal(size=(S, Hh, D))
    p = rng.integers(0, 5000, size=S)
    cos, sin = oracle.rope_cos_sin(np.stack([p, p, p]), D, theta, (24, 20, 20))
    y = oracle.apply_rope(x, cos, sin)
    half = D // 2
    omega = theta ** (-np.arange(half) * 2.0 / D)
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * p[:, None, None] * omega[None, None, :])
    np.testing.assert_allclose(y[..., :half], z.real, atol=1e-12)
    np.testing.assert_allclose(y[..., half:], z.imag, atol=1e-12)


def test_rope_relative_position_property():
    rng = np.random.default_rng(5)
    D = 128
    q = rng.normal(size=(1, 1, D)); k = rng.normal(size=(1, 1, D))

    def dot(pq, pk):
        pos = np.array([[pq, pk]] * 3)
        cos, sin = oracle.rope_cos_sin(pos, D, 5e6, (24, 20, 20))
        rq = oracle.apply_rope(q, cos[:1], sin[:1])
        rk = oracle.apply_rope(k, cos[1:], sin[1:])
        return float(np.sum(rq * rk))

    assert dot(100, 40) == pytest.approx(dot(1060, 1000), rel=1e-9, abs=1e-9)
    assert dot(7, 7) == pytest.approx(float(np.sum(q * k)), rel=1e-12)


def test_rope_each_axis_drives_its_slots():
    """Moving only the H axis rotates exactly the H slots; likewise W and T."""
    D = 128
    half = D // 2
    base = np.array([[10], [20], [30]])
    table = _slot_fixture("mrope_slots_d128.txt")
    cos0, sin0 = oracle.rope_cos_sin(base, D, 5e6, (24, 20, 20))
    for a, key in enumerate("THW"):
        moved = base.copy(); moved[a, 0] += 9
        cos1, _ = oracle.rope_cos_sin(moved, D, 5e6, (24, 20, 20))
        changed = np.flatnonzero(np.abs(cos1[0, :half] - cos0[0, :half]) > 0)
        assert changed.tolist() == table[key]


# ---------------------------------------------------------------- attention

def test_attention_equal_keys_gives_prefix_mean():
    rng = np.random.default_rng(6)
    S, Hq, Hkv, D = 17, 4, 2, 16
    q = rng.normal(size=(S, Hq, D))
    k = np.broadcast_to(rng.normal(size=(1, Hkv, D)), (S, Hkv, D)).copy()
    v = rng.normal(size=(S, Hkv, D))
    out = oracle.causal_gqa_attention(q, k, v)
    prefix = np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None, None]
    for h in range(Hq):
        np.testing.assert_allclose(out[:, h], prefix[:, h // 2], rtol=1e-12, atol=1e-12)


def test_attention_single_token_returns_value():
    rng = np.random.default_rng(7)
    q = rng.normal(size=(1, 8, 32)); k = rng.normal(size=(1, 1, 32)); v = rng.normal(size=(1, 1, 32))
    out = oracle.causal_gqa_attention(q, k, v)
    for h in range(8):
        np.testing.assert_allclose(out[0, h], v[0, 0], rtol=1e-14)


@pytest.mark.parametrize("S,Hq,Hkv,D", [(37, 8, 2, 32), (70, 4, 1, 64), (9, 6, 3, 128)])
def test_attention_matches_torch_sdpa(S, Hq, Hkv, D):
    rng = np.random.default_rng(S)
    q = rng.normal(size=(S, Hq, D)); k = rng.normal(size=(S, Hkv, D)); v = rng.normal(size=(S, Hkv, D))
    tq, tk, tv = (torch.from_numpy(a).transpose(0, 1)[None] for a in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)[0].transpose(0, 1)
    np.testing.assert_allclose(oracle.causal_gqa_attention(q, k, v, block=16), ref.numpy(), rtol=1e-10, atol=1e-12)


def test_attention_row_subset_and_causality():
    rng = np.random.default_rng(8)
    S, Hq, Hkv, D = 40, 4, 2, 16
    q = rng.normal(size=(S, Hq, D)); k = rng.normal(size=(S, Hkv, D)); v = rng.normal(size=(S, Hkv, D))
    full = oracle.causal_gqa_attention(q, k, v)
    rows = np.array([0, 5, 19, 39])
    np.testing.assert_allclose(oracle.causal_gqa_attention(q, k, v, rows=rows), full[rows], rtol=1e-13, atol=1e-14)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[25:] += 3; k2[25:] -= 2; v2[25:] *= 5
    out2 = oracle.causal_gqa_attention(q2, k2, v2)
    assert np.array_equal(out2[:25], full[:25])


def test_attention_dominant_logit_selects_key():
    S, D = 6, 8
    q = np.zeros((S, 1, D)); k = np.zeros((S, 1, D)); v = np.arange(S * D, dtype=float).reshape(S, 1, D)
    k[2, 0, 0] = 1.0
    q[:, 0, 0] = 400.0   # logit 400/sqrt(8) on key 2, 0 elsewhere
    out = oracle.causal_gqa_attention(q, k, v)
    np.testing.assert_allclose(out[3:, 0], np.broadcast_to(v[2, 0], (3, D)), rtol=1e-12)
    np.testing.assert_allclose(out[0, 0], v[0, 0])


# ---------------------------------------------------------------- SiLU / layer

def test_silu_closed_form():
    from scipy.special import expit
    z = np.linspace(-30, 30, 241)
    np.testing.assert_allclose(oracle.silu(z), z * expit(z), rtol=1e-13, atol=1e-300)
    assert oracle.silu(0.0) == 0.0
    np.testing.assert_allclose(oracle.silu(torch.linspace(-8, 8, 33, dtype=torch.float64).numpy()),
                               F.silu(torch.linspace(-8, 8, 33, dtype=torch.float64)).numpy(), rtol=1e-13)


def _tiny_dims(Hq=4, Hkv=2, D=16, H=48, I=80):
    return ModelDims(hidden=H, n_heads=Hq, n_kv_heads=Hkv, head_dim=D, intermediate=I,
                     rms_eps=1e-6, rope_theta=1e4, mrope_section=(24, 20, 20))


def _rand_layer(dims, rng, std=0.2):
    H, D, Hq, Hkv, I = dims.hidden, dims.head_dim, dims.n_heads, dims.n_kv_heads, dims.intermediate
    n = lambda *s: rng.normal(size=s) * std
    u = lambda *s: rng.uniform(0.5, 1.5, size=s)
    return LayerWeights(ln_in=u(H), w_q=n(Hq * D, H), w_k=n(Hkv * D, H), w_v=n(Hkv * D, H),
                        q_norm=u(D), k_norm=u(D), w_o=n(H, Hq * D), ln_post=u(H),
                        w_gate=n(I, H), w_up=n(I, H), w_down=n(H, I))


def _torch_layer(h, w, p, dims):
    """Independent composition from torch library routines; rotary as complex rotation.

    Valid for text-only positions (all three axes equal p)."""
    S, H = h.shape
    D, Hq, Hkv, eps = dims.head_dim, dims.n_heads, dims.n_kv_heads, dims.rms_eps
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    x = T(h)
    u = F.rms_norm(x, (H,), weight=T(w.ln_in), eps=eps)
    q = F.rms_norm(F.linear(u, T(w.w_q)).view(S, Hq, D), (D,), weight=T(w.q_norm), eps=eps)
    k = F.rms_norm(F.linear(u, T(w.w_k)).view(S, Hkv, D), (D,), weight=T(w.k_norm), eps=eps)
    v = F.linear(u, T(w.w_v)).view(S, Hkv, D)
    half = D // 2
    omega = dims.rope_theta ** (-torch.arange(half, dtype=torch.float64) * 2.0 / D)
    rot = torch.polar(torch.ones(S, half, dtype=torch.float64), T(p).double()[:, None] * omega[None, :])

    def rope(t):
        z = torch.complex(t[..., :half], t[..., half:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    q, k = rope(q), rope(k)
    o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                       v.transpose(0, 1)[None], is_causal=True, enable_gqa=True)
    o = o[0].transpose(0, 1).reshape(S, Hq * D)
    h1 = x + F.linear(o, T(w.w_o))
    u2 = F.rms_norm(h1, (H,), weight=T(w.ln_post), eps=eps)
    return (h1 + F.linear(F.silu(F.linear(u2, T(w.w_gate))) * F.linear(u2, T(w.w_up)), T(w.w_down))).numpy()


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (8, 2), (4, 1)])
def test_decoder_layer_matches_library_composition(Hq, Hkv):
    rng = np.random.default_rng(10 + Hq + Hkv)
    dims = _tiny_dims(Hq=Hq, Hkv=Hkv)
    S = 23
    w = _rand_layer(dims, rng)
    h = rng.normal(size=(S, dims.hidden))
    p = np.arange(S) * 3 + 5
    cos, sin = oracle.rope_cos_sin(np.stack([p, p, p]), dims.head_dim, dims.rope_theta, dims.mrope_section)
    got = oracle.decoder_layer(h, w, cos, sin, dims)
    np.testing.assert_allclose(got, _torch_layer(h, w, p, dims), rtol=1e-10, atol=1e-10)


def test_decoder_layer_zero_projections_is_identity():
    rng = np.random.default_rng(11)
    dims = _tiny_dims()
    w = _rand_layer(dims, rng)
    w.w_o[:] = 0.0
    w.w_down[:] = 0.0
    h = rng.normal(size=(9, dims.hidden))
    cos, sin = oracle.rope_cos_sin(np.zeros((3, 9), int), dims.head_dim, dims.rope_theta, dims.mrope_section)
    assert np.array_equal(oracle.decoder_layer(h, w, cos, sin, dims), h)


def test_decoder_layer_zero_value_is_mlp_only():
    """W_v = 0 -> attention contributes nothing; output = h + MLP(rms(h, post gain))."""
    rng = np.random.default_rng(12)
    dims = _tiny_dims()
    w = _rand_layer(dims, rng)
    w.w_v[:] = 0.0
    h = rng.normal(size=(9, dims.hidden))
    cos, sin = oracle.rope_cos_sin(np.zeros((3, 9), int), dims.head_dim, dims.rope_theta, dims.mrope_section)
    T = torch.from_numpy
    u2 = F.rms_norm(T(h), (dims.hidden,), weight=T(w.ln_post), eps=dims.rms_eps)
    mlp = F.linear(F.silu(F.linear(u2, T(w.w_gate))) * F.linear(u2, T(w.w_up)), T(w.w_down)).numpy()
    np.testing.assert_allclose(oracle.decoder_layer(h, w, cos, sin, dims), h + mlp, rtol=1e-12, atol=1e-12)


def test_decoder_layer_row_subset():
    rng = np.random.default_rng(13)
    dims = _tiny_dims()
    w = _rand_layer(dims, rng)
    S = 30
    h = rng.normal(size=(S, dims.hidden))
    pos = rng.integers(0, 100, size=(3, S))
    cos, sin = oracle.rope_cos_sin(pos, dims.head_dim, dims.rope_theta, dims.mrope_section)
    full = oracle.decoder_layer(h, w, cos, sin, dims)
    rows = np.array([0, 3, 17, 29])
    np.testing.assert_allclose(oracle.decoder_layer(h, w, cos, sin, dims, rows=rows), full[rows],
                               rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- DeepStack / encode

def test_deepstack_worked_example():
    kv = {}
    for ln in _lines("deepstack_worked.txt"):
        k, v = ln.split(":")
        kv[k.strip()] = v.strip()
    mask = np.array([int(x) for x in kv["mask"].split()])
    mat = lambda s: np.array([_vec(r) for r in s.split("|")])
    got = oracle.deepstack_add(mat(kv["hidden"]), mask, mat(kv["feature"]))
    assert np.array_equal(got, mat(kv["expected"]))


def test_deepstack_equals_dense_buffer_form():
    """vLLM Qwen3-VL page: features live in a dense [S, H] buffer, zero off the
    visual rows, added to every row after the layer; same as the masked add."""
    rng = np.random.default_rng(14)
    S, H = 12, 8
    mask = rng.integers(0, 2, size=S).astype(bool)
    h = rng.normal(size=(S, H)); feat = rng.normal(size=(int(mask.sum()), H))
    dense = np.zeros((S, H)); dense[mask] = feat
    np.testing.assert_allclose(oracle.deepstack_add(h, mask, feat), h + dense, rtol=0, atol=0)
    with pytest.raises(ValueError):
        oracle.deepstack_add(h, mask, feat[:-1])


def _stack(dims, n, rng):
    return [_rand_layer(dims, rng) for _ in range(n)]


def test_encode_structure_and_deepstack_placement():
    rng = np.random.default_rng(15)
    dims = _tiny_dims()
    S = 20
    layers = _stack(dims, 3, rng)
    e = rng.normal(size=(S, dims.hidden))
    pos = rng.integers(0, 50, size=(3, S))
    mask = np.zeros(S, bool); mask[6:14] = True
    ds = [rng.normal(size=(8, dims.hidden)) for _ in range(5)]   # more levels than layers: extras unused
    assert np.array_equal(oracle.encode(e, pos, layers, dims, n_layers=0), e)
    cos, sin = oracle.rope_cos_sin(pos, dims.head_dim, dims.rope_theta, dims.mrope_section)
    h = e
    for l in range(3):
        h = oracle.decoder_layer(h, layers[l], cos, sin, dims)
        h = h.copy(); h[mask] += ds[l]      # after the layer's MLP residual, before the next layer
    got = oracle.encode(e, pos, layers, dims, visual_mask=mask, deepstack=ds)
    np.testing.assert_allclose(got, h, rtol=1e-13, atol=1e-13)
    # without DeepStack the result differs (the levels are really injected)
    assert not np.allclose(oracle.encode(e, pos, layers, dims), got)
    states = oracle.encode(e, pos, layers, dims, visual_mask=mask, deepstack=ds, return_all=True)
    assert len(states) == 4 and np.array_equal(states[-1], got)


def test_encode_is_causal_bitwise():
    rng = np.random.default_rng(16)
    dims = _tiny_dims()
    S, cut = 24, 11
    layers = _stack(dims, 2, rng)
    e = rng.normal(size=(S, dims.hidden))
    pos = rng.integers(0, 50, size=(3, S))
    mask = np.zeros(S, bool); mask[5:20] = True
    ds = [rng.normal(size=(15, dims.hidden)) for _ in range(2)]
    a = oracle.encode(e, pos, layers, dims, visual_mask=mask, deepstack=ds)
    e2 = e.copy(); e2[cut:] += 1.5
    ds2 = [d.copy() for d in ds]
    for d in ds2:
        d[cut - 5:] -= 2.0          # visual rows at tokens >= cut
    pos2 = pos.copy(); pos2[:, cut:] += 7
    b = oracle.encode(e2, pos2, layers, dims, visual_mask=mask, deepstack=ds2)
    assert np.array_equal(a[:cut], b[:cut])
    assert not np.allclose(a[cut:], b[cut:])


# ---------------------------------------------------------------- shapes / positions

def test_parameter_count_reproduces_footprint():
    """50 full-width layers in bf16, plus the vision tower (~1.2 GB) and a
    151936 x 5120 embedding table, come to the pages' ~51.5 GB."""
    dims = ModelDims(hidden=5120, n_heads=64, n_kv_heads=8, head_dim=128, intermediate=25600)
    per_layer = oracle.layer_param_count(dims)
    assert per_layer - (2 * 5120 + 2 * 128) == 487_587_840
    total_gb = (50 * per_layer * 2 + 151936 * 5120 * 2) / 1e9 + 1.2
    assert abs(total_gb - 51.5) < 0.1


def test_positions_worked_examples_and_synth_recipe():
    from multimodal_encoder_prefill_amd import synth
    rows = [[p.strip() for p in ln.split("|")] for ln in _lines("positions_workloads.txt")]
    for key in sorted({r[0] for r in rows}):
        wl = synth.WORKLOADS[key]
        ref = oracle.text_and_grid_positions(wl.segments)
        assert ref.shape == (3, wl.seq)
        assert np.array_equal(synth.positions(wl), ref)
        for r in rows:
            if r[0] == key:
                tok = int(r[1])
                assert ref[:, tok].tolist() == [int(x) for x in r[2].split()], (key, tok)


# ---------------------------------------------------------------- token front end

IMG_ID, VID_ID = 151655, 151656


def _ids_from_types(types, seed=0):
    """Token ids of the given types: text ids drawn below the special ids."""
    rng = np.random.default_rng(seed)
    types = np.asarray(types)
    ids = rng.integers(0, 151000, size=len(types))
    ids[types == 1] = IMG_ID
    ids[types == 2] = VID_ID
    return ids


def test_rope_index_worked_example():
    rows = {k: v for k, v in (ln.split("|") for ln in _lines("rope_index_mixed.txt"))}
    rows = {k.strip(): v.split() for k, v in rows.items()}
    types = [int(x) for x in rows["types"]]
    ids = _ids_from_types(types)
    pos, delta = oracle.frontend.rope_index(ids, IMG_ID, VID_ID,
                                            [[int(x) for x in rows["image_grid"]]],
                                            [[int(x) for x in rows["video_grid"]]],
                                            int(rows["merge"][0]))
    want = np.array([[int(x) for x in rows[a]] for a in ("t", "h", "w")])
    assert np.array_equal(pos, want)
    assert delta == int(rows["delta"][0])


def test_rope_index_text_only_is_a_ramp():
    ids = _ids_from_types(np.zeros(37, dtype=int), seed=3)
    pos, delta = oracle.frontend.rope_index(ids, IMG_ID, VID_ID, None, None, 2)
    assert np.array_equal(pos, np.tile(np.arange(37), (3, 1)))
    assert delta == 0


def test_rope_index_agrees_with_segment_rule_on_workloads():
    # two formulations of the page's rule: from token ids (runs of equal
    # type) and from the workloads' segment lists
    from multimodal_encoder_prefill_amd import synth
    for name in ("image_s2048_l4", "image_s4096_l50", "video_s16384_l50"):
        wl = synth.WORKLOADS[name]
        types, igrids = [], []
        for kind, spec in wl.segments:
            if kind == "text":
                types += [0] * int(spec)
            else:
                t, h, w = (int(x) for x in spec)
                types += [1] * (t * h * w)
                igrids.append((t, 2 * h, 2 * w))
        ids = _ids_from_types(types, seed=5)
        pos, delta = oracle.frontend.rope_index(ids, IMG_ID, VID_ID, igrids, None, 2)
        ref = oracle.text_and_grid_positions(wl.segments)
        assert np.array_equal(pos, ref)
        assert delta == int(ref.max()) + 1 - ref.shape[1]


def test_rope_index_rejects_runs_that_do_not_fit_a_grid():
    ids = _ids_from_types([0, 1, 1, 1, 0])
    with pytest.raises(ValueError):  # 3 tokens, grid holds 4
        oracle.frontend.rope_index(ids, IMG_ID, VID_ID, [[1, 4, 4]], None, 2)
    with pytest.raises(ValueError):  # no grid at all
        oracle.frontend.rope_index(ids, IMG_ID, VID_ID, None, None, 2)
    # adjacent frames with no text between them are one run: it holds two
    # frames' tokens, more than the one-frame grid it takes
    ids = _ids_from_types([0] + [2] * 8 + [0])
    with pytest.raises(ValueError):
        oracle.frontend.rope_index(ids, IMG_ID, VID_ID, None, [[2, 4, 4]], 2)


def test_embed_and_scatter_places_rows():
    # a table whose row i is filled with i identifies every gathered row
    vocab, hid = 151936, 8
    table = np.repeat(np.arange(vocab, dtype=np.float64)[:, None], hid, axis=1)
    types = [0, 1, 1, 0, 2, 0, 1]
    ids = _ids_from_types(types, seed=7)
    img = -1.0 - np.arange(3 * hid, dtype=np.float64).reshape(3, hid)
    vid = -100.0 - np.arange(hid, dtype=np.float64)[None, :]
    out = oracle.frontend.embed_and_scatter(table, ids, IMG_ID, VID_ID, img, vid)
    for t in (0, 3, 5):
        assert np.all(out[t] == ids[t])
    np.testing.assert_array_equal(out[[1, 2, 6]], img)
    np.testing.assert_array_equal(out[4], vid[0])
    with pytest.raises(ValueError):
        oracle.frontend.embed_and_scatter(table, ids, IMG_ID, VID_ID, img[:2], None)


def test_aggregate_deepstack_joint_order():
    S, hid = 12, 4
    image_mask = np.zeros(S, bool)
    video_mask = np.zeros(S, bool)
    image_mask[[1, 2, 7]] = True
    video_mask[[4, 5, 9, 10]] = True
    rng = np.random.default_rng(11)
    img = [rng.normal(size=(3, hid)) for _ in range(3)]
    vid = [rng.normal(size=(4, hid)) for _ in range(3)]
    vis, levels = oracle.frontend.aggregate_deepstack(image_mask, video_mask, img, vid)
    assert np.array_equal(np.nonzero(vis)[0], [1, 2, 4, 5, 7, 9, 10])
    for l in range(3):
        # the joint rows, put back on their tokens, give each modality's rows
        full = np.zeros((S, hid))
        full[vis] = levels[l]
        np.testing.assert_array_equal(full[image_mask], img[l])
        np.testing.assert_array_equal(full[video_mask], vid[l])
    m, lv = oracle.frontend.aggregate_deepstack(image_mask, None, img, None)
    assert np.array_equal(m, image_mask) and lv is img
