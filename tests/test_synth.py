"""Seeded input generator: determinism, shapes, distributions, bf16 storage."""

import numpy as np
import torch

from multimodal_encoder_prefill_amd import synth


def test_layer_weights_deterministic_and_shaped():
    wl = synth.WORKLOADS["tiny"]
    a = synth.layer_weights(wl, 1)
    b = synth.layer_weights(wl, 1)
    c = synth.layer_weights(wl, 0)
    for name, shape in synth.layer_shapes(wl.dims).items():
        assert a[name].shape == shape and a[name].dtype == torch.bfloat16
        assert torch.equal(a[name], b[name])
        assert not torch.equal(a[name], c[name])


def test_distributions():
    wl = synth.WORKLOADS["tiny"]
    w = synth.layer_weights(wl, 0)
    assert abs(w["w_gate"].float().std().item() - 0.02) < 0.001
    g = w["ln_in"].float()
    assert 0.5 <= g.min().item() and g.max().item() <= 1.5
    e = synth.embeddings(wl).float()
    assert abs(e.std().item() - 1.0) < 0.05 and e.shape == (64, 256)


def test_masks_and_counts():
    for wl in synth.WORKLOADS.values():
        m = synth.visual_mask(wl)
        assert m.shape == (wl.seq,) and int(m.sum()) == wl.n_vis
        p = synth.positions(wl)
        assert p.shape == (3, wl.seq) and p.dtype == np.int32
    wl = synth.WORKLOADS["image_s4096_l50"]
    m = synth.visual_mask(wl)
    assert m[:1024].sum() == 0 and m[1024:3072].all() and m[3072:].sum() == 0
