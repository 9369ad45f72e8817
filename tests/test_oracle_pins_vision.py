"""Pins of the vision-tower oracle against things other than itself: torch's
layer_norm, gelu (both forms), conv3d and scaled_dot_product_attention,
complex-number rotation, closed forms of bilinear interpolation and of the
2-D rotary angles, and structural properties (segments do not interact,
DeepStack taken after the listed blocks)."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import vision as V

TINY = V.VisionDims(hidden=48, n_heads=2, intermediate=40, depth=3, patch=2, temporal_patch=2,
                    in_channels=3, merge=2, out_hidden=32, pos_side=6, deepstack=(0, 2))


def _t(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64))


def test_layer_norm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(7, 48)) * 3 + 1
    w, b = rng.uniform(0.5, 1.5, 48), rng.normal(size=48)
    ref = F.layer_norm(_t(x), (48,), _t(w), _t(b), eps=1e-6).numpy()
    np.testing.assert_allclose(V.layer_norm(x, w, b), ref, rtol=1e-12, atol=1e-12)


def test_gelu_forms_match_torch():
    x = np.linspace(-8, 8, 401)
    np.testing.assert_allclose(V.gelu_tanh(x), F.gelu(_t(x), approximate="tanh").numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(V.gelu_erf(x), F.gelu(_t(x)).numpy(), rtol=1e-12, atol=1e-14)
    # the two forms are different functions
    assert np.max(np.abs(V.gelu_tanh(x) - V.gelu_erf(x))) > 1e-4


def test_patch_embed_is_the_strided_conv3d():
    rng = np.random.default_rng(1)
    C, T, P, hid, n = 3, 2, 4, 5, 6
    x = rng.normal(size=(n, C * T * P * P))
    w = rng.normal(size=(hid, C, T, P, P))
    b = rng.normal(size=hid)
    ref = F.conv3d(_t(x).view(-1, C, T, P, P), _t(w), _t(b), stride=(T, P, P)).view(-1, hid).numpy()
    np.testing.assert_allclose(V.patch_embed(x, w, b), ref, rtol=1e-12, atol=1e-12)


def test_pos_embed_identity_on_the_table_grid():
    S = 6
    table = np.random.default_rng(2).normal(size=(S * S, 4))
    got = V.pos_embed_interpolate(table, [(1, S, S)], S, 1)
    np.testing.assert_allclose(got, table, rtol=0, atol=1e-12)


def test_pos_embed_bilinear_of_a_linear_table_and_block_order():
    # table value = (row, col, 1) at table cell (row, col): bilinear interpolation
    # returns the sampling point exactly, which also names the patch it belongs to
    S, t, h, w, m = 6, 2, 4, 8, 2
    rr, cc = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    table = np.stack([rr.ravel(), cc.ravel(), np.ones(S * S)], axis=1).astype(np.float64)
    got = V.pos_embed_interpolate(table, [(t, h, w)], S, m)
    k = 0
    for f in range(t):
        for br in range(h // m):
            for bc in range(w // m):
                for ir in range(m):
                    for ic in range(m):
                        r, c = br * m + ir, bc * m + ic
                        want = [r * (S - 1) / (h - 1), c * (S - 1) / (w - 1), 1.0]
                        np.testing.assert_allclose(got[k], want, rtol=1e-6, atol=1e-6)
                        k += 1
    assert k == got.shape[0]


def test_rotary_angles_worked_example():
    # head_dim 8: half 4, frequencies theta^0 = 1 and theta^(-2/4) = 1/100;
    # grid 1x4x4 with merge 2: token 5 is in block (0, 1) at (ir, ic) = (0, 1),
    # i.e. row 0, column 3
    ang = V.rotary_angles([(1, 4, 4)], 8, 2)
    np.testing.assert_allclose(ang[5], [0, 0, 3, 0.03, 0, 0, 3, 0.03], rtol=1e-12)
    np.testing.assert_allclose(ang[10], [3, 0.03, 0, 0, 3, 0.03, 0, 0], rtol=1e-12)   # row 3, col 0


def test_rope_is_complex_rotation_of_half_pairs():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(5, 2, 8))
    ang = rng.uniform(-3, 3, size=(5, 8))
    ang[:, 4:] = ang[:, :4]
    z = (x[..., :4] + 1j * x[..., 4:]) * np.exp(1j * ang[:, None, :4])
    got = V.rope(x, ang)
    np.testing.assert_allclose(got[..., :4], z.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got[..., 4:], z.imag, rtol=1e-12, atol=1e-12)


def test_segment_attention_matches_torch_sdpa_and_segments_are_independent():
    rng = np.random.default_rng(4)
    n, H, D = 20, 2, 8
    q, k, v = (rng.normal(size=(n, H, D)) for _ in range(3))
    segs = [(0, 7), (7, 16), (16, 20)]
    got = V.segment_attention(q, k, v, segs).reshape(n, H, D)
    for s, e in segs:
        ref = F.scaled_dot_product_attention(_t(q[s:e]).transpose(0, 1), _t(k[s:e]).transpose(0, 1),
                                             _t(v[s:e]).transpose(0, 1)).transpose(0, 1).numpy()
        np.testing.assert_allclose(got[s:e], ref, rtol=1e-10, atol=1e-12)
    k2 = k.copy()
    k2[7:16] += rng.normal(size=(9, H, D))
    got2 = V.segment_attention(q, k2, v, segs).reshape(n, H, D)
    assert np.array_equal(got2[:7], got[:7]) and np.array_equal(got2[16:], got[16:])
    assert not np.allclose(got2[7:16], got[7:16])


def _block_params(rng, d):
    H, I = d.hidden, d.intermediate
    g = lambda *s: rng.normal(size=s) * 0.2
    return {"norm1_w": rng.uniform(0.5, 1.5, H), "norm1_b": g(H), "qkv_w": g(3 * H, H), "qkv_b": g(3 * H),
            "proj_w": g(H, H), "proj_b": g(H), "norm2_w": rng.uniform(0.5, 1.5, H), "norm2_b": g(H),
            "fc1_w": g(I, H), "fc1_b": g(I), "fc2_w": g(H, I), "fc2_b": g(H)}


def test_block_matches_torch_composition():
    rng = np.random.default_rng(5)
    d = TINY
    grids = [(1, 4, 4), (2, 2, 4)]
    n = 16 + 16
    x = rng.normal(size=(n, d.hidden))
    p = _block_params(rng, d)
    ang = V.rotary_angles(grids, d.head_dim, d.merge)
    segs = V.segments(grids)
    got = V.block(x, p, d, ang, segs)
    T = {k: _t(v) for k, v in p.items()}
    X = _t(x)
    H, Dh = d.n_heads, d.head_dim
    u = F.layer_norm(X, (d.hidden,), T["norm1_w"], T["norm1_b"], eps=1e-6)
    qkv = F.linear(u, T["qkv_w"], T["qkv_b"]).view(n, 3, H, Dh)
    a = _t(ang)[:, None, : Dh // 2]

    def rot(z):  # complex rotation of the (d, d + D/2) pairs
        c = torch.complex(z[..., : Dh // 2], z[..., Dh // 2:]) * torch.exp(1j * a)
        return torch.cat([c.real, c.imag], dim=-1)
    q, k, v = rot(qkv[:, 0]), rot(qkv[:, 1]), qkv[:, 2]
    outs = []
    for s, e in segs:
        outs.append(F.scaled_dot_product_attention(q[s:e].transpose(0, 1), k[s:e].transpose(0, 1),
                                                   v[s:e].transpose(0, 1)).transpose(0, 1))
    att = torch.cat(outs).reshape(n, -1)
    X = X + F.linear(att, T["proj_w"], T["proj_b"])
    u = F.layer_norm(X, (d.hidden,), T["norm2_w"], T["norm2_b"], eps=1e-6)
    X = X + F.linear(F.gelu(F.linear(u, T["fc1_w"], T["fc1_b"]), approximate="tanh"), T["fc2_w"], T["fc2_b"])
    np.testing.assert_allclose(got, X.numpy(), rtol=1e-10, atol=1e-10)


def test_mergers_match_torch_composition():
    rng = np.random.default_rng(6)
    d = TINY
    x = rng.normal(size=(16, d.hidden))
    mh = d.merged_hidden
    for post in (False, True):
        nd = mh if post else d.hidden
        p = {"norm_w": rng.uniform(0.5, 1.5, nd), "norm_b": rng.normal(size=nd),
             "fc1_w": rng.normal(size=(mh, mh)) * 0.1, "fc1_b": rng.normal(size=mh),
             "fc2_w": rng.normal(size=(d.out_hidden, mh)) * 0.1, "fc2_b": rng.normal(size=d.out_hidden)}
        T = {k: _t(v) for k, v in p.items()}
        X = _t(x)
        if post:
            u = F.layer_norm(X.view(-1, mh), (mh,), T["norm_w"], T["norm_b"], eps=1e-6)
        else:
            u = F.layer_norm(X, (d.hidden,), T["norm_w"], T["norm_b"], eps=1e-6).view(-1, mh)
        ref = F.linear(F.gelu(F.linear(u, T["fc1_w"], T["fc1_b"])), T["fc2_w"], T["fc2_b"]).numpy()
        np.testing.assert_allclose(V.merger(x, p, d, post), ref, rtol=1e-10, atol=1e-10)


def test_forward_structure_deepstack_after_listed_blocks():
    rng = np.random.default_rng(7)
    d = TINY
    grids = [(1, 4, 4)]
    n = 16
    px = rng.normal(size=(n, d.patch_dim))
    mh = d.merged_hidden

    def mp(post):
        nd = mh if post else d.hidden
        return {"norm_w": rng.uniform(0.5, 1.5, nd), "norm_b": rng.normal(size=nd),
                "fc1_w": rng.normal(size=(mh, mh)) * 0.1, "fc1_b": rng.normal(size=mh),
                "fc2_w": rng.normal(size=(d.out_hidden, mh)) * 0.1, "fc2_b": rng.normal(size=d.out_hidden)}
    w = {"patch_w": rng.normal(size=(d.hidden, d.in_channels, d.temporal_patch, d.patch, d.patch)) * 0.1,
         "patch_b": rng.normal(size=d.hidden), "pos_table": rng.normal(size=(d.pos_side ** 2, d.hidden)),
         "blocks": [_block_params(rng, d) for _ in range(d.depth)], "merger": mp(False),
         "deepstack": [mp(True) for _ in d.deepstack]}
    out, ds, states = V.forward(px, grids, w, d, return_blocks=True)
    assert out.shape == (n // 4, d.out_hidden) and len(ds) == 2
    np.testing.assert_allclose(ds[0], V.merger(states[1], w["deepstack"][0], d, True), rtol=1e-12)
    np.testing.assert_allclose(ds[1], V.merger(states[3], w["deepstack"][1], d, True), rtol=1e-12)
    np.testing.assert_allclose(out, V.merger(states[3], w["merger"], d, False), rtol=1e-12)
    x0 = V.patch_embed(px, w["patch_w"], w["patch_b"]) + V.pos_embed_interpolate(w["pos_table"], grids, d.pos_side, 2)
    np.testing.assert_allclose(states[0], x0, rtol=1e-12)
