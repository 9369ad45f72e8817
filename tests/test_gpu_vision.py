"""Vision tower of the HIP path against the float64 oracle (oracle.vision).

Bars from the arithmetic, as for the decoder: a step that accumulates in
fp32 and rounds its output to bf16 once (LayerNorm, the biased linears with
their activation or residual) agrees with the oracle to rel-L2 <= 4e-3; the
patch embedding rounds twice (the biased GEMM, then the position-table add):
6e-3; a merger three times, two of them feeding a GEMM: 1e-2; attention
rounds its probabilities to bf16 as well: 8e-3 (and 3e-2 for any single
(patch, head) row). A block fed the GPU's own bf16 input (teacher-forced)
agrees to <= 2e-2; the free-running tower to <= 5e-2 at its outputs. Grids mix images and multi-frame videos so the
per-frame attention segments, the merge-block order and the position-table
interpolation are all exercised; frames are checked to be independent
bitwise.
"""

import numpy as np
import pytest
import torch

from oracle import vision as OV
from multimodal_encoder_prefill_amd import binding as b
from multimodal_encoder_prefill_amd import synth
from helpers import f64, report, report_rows, perm16_tokens

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _odims(vd, depth=None):
    return OV.VisionDims(hidden=vd.hidden, n_heads=vd.n_heads, intermediate=vd.mlp_width,
                         depth=vd.depth if depth is None else depth, patch=vd.patch,
                         temporal_patch=vd.temporal_patch, in_channels=vd.in_channels,
                         merge=vd.merge, out_hidden=vd.out_hidden, pos_side=vd.pos_side,
                         deepstack=tuple(vd.deepstack))


def _oblock(p, width):
    o = {k: f64(v) for k, v in p.items()}
    o["fc1_w"], o["fc1_b"], o["fc2_w"] = o["fc1_w"][:width], o["fc1_b"][:width], o["fc2_w"][:, :width]
    return o


def _omerger(m):
    return {k: f64(v) for k, v in m.items()}


def _setup(vd, grids, seed=0):
    w = synth.vision_weights(vd, seed, DEV)
    n = int(sum(t * h * ww for t, h, ww in grids))
    px = synth.vision_pixels(n, vd, seed, DEV)
    cfg = b.vision_config(vd)
    nb = b.vision_workspace_bytes(cfg, n)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    return w, b.VisionTables(w), px, n, cfg, ws, nb


GRIDS_TINY = [(1, 8, 8), (2, 4, 8), (1, 6, 4)]
GRIDS_FULL = [(1, 32, 32), (2, 16, 16)]


@pytest.mark.parametrize("offset", [0.5, 300.0, -2000.0])
def test_layer_norm_matches_oracle(offset):
    """Rows of N(offset, 4): the large offsets check that the statistics do
    not cancel against a mean far from zero (bf16 keeps only ~3 significant
    digits of the offset, so the rows' spread survives as bf16 steps)."""
    for dim in (576, 1152, 4608):
        g = torch.Generator(device=DEV).manual_seed(dim)
        x = (torch.randn(257, dim, generator=g, device=DEV) * 2 + offset).to(torch.bfloat16)
        w = (0.5 + torch.rand(dim, generator=g, device=DEV)).to(torch.bfloat16)
        bb = (0.1 * torch.randn(dim, generator=g, device=DEV)).to(torch.bfloat16)
        y = torch.empty_like(x)
        b.layer_norm(x, w, bb, y, 257, dim)
        torch.cuda.synchronize()
        ref = OV.layer_norm(f64(x), f64(w), f64(bb))
        assert report(f"layer_norm dim {dim}", f64(y), ref)[0] <= 4e-3
        # one bf16 rounding: every element within half an ulp of the fp32 result plus slack
        assert np.max(np.abs(f64(y) - ref) / (np.abs(ref) + 1e-2)) < 2e-2


@pytest.mark.parametrize("act", [0, 1, 2, "res"])
def test_linear_bias_matches_oracle(act):
    m, n, k = 300, 576, 1152
    g = torch.Generator(device=DEV).manual_seed(7)
    a = torch.randn(m, k, generator=g, device=DEV).to(torch.bfloat16)
    w = (0.03 * torch.randn(n, k, generator=g, device=DEV)).to(torch.bfloat16)
    bias = (0.5 * torch.randn(n, generator=g, device=DEV)).to(torch.bfloat16)
    r = torch.randn(m, n, generator=g, device=DEV).to(torch.bfloat16)
    c = r.clone() if act == "res" else torch.empty(m, n, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(b.linear_workspace_bytes(), dtype=torch.uint8, device=DEV)
    b.linear_bias(a, w, bias, c, m, n, k, act=0 if act == "res" else act,
                  residual=c if act == "res" else None, workspace=ws)
    torch.cuda.synchronize()
    y = OV.linear(f64(a), f64(w), f64(bias))
    ref = {0: y, 1: OV.gelu_tanh(y), 2: OV.gelu_erf(y), "res": y + f64(r)}[act]
    assert report(f"linear_bias act={act}", f64(c), ref)[0] <= 4e-3


@pytest.mark.parametrize("grids,heads,hd", [(GRIDS_TINY, 8, 72), (GRIDS_FULL, 16, 72),
                                           ([(1, 64, 128)], 16, 72), (GRIDS_TINY, 4, 128),
                                           (GRIDS_TINY, 4, 80), (GRIDS_TINY, 4, 96)])
def test_vision_attention_per_frame(grids, heads, hd):
    """The per-frame attention step on its own: every (patch, head) row
    against the oracle's segment attention, frames as the grids cut them (the
    benched single 64 x 128-patch frame included)."""
    n = int(sum(t * h * w for t, h, w in grids))
    print(f"vision attention n={n} heads={heads} head_dim={hd} grids={grids}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(n + hd)
    q = torch.randn(n, heads, hd, generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn(n, heads, hd, generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn(n, heads, hd, generator=g, device=DEV).to(torch.bfloat16)
    sp = b.seq_pad(n)
    q_l = torch.zeros(n, heads, 128, dtype=torch.bfloat16, device=DEV)
    q_l[:, :, :hd] = q
    k_l = torch.zeros(heads, sp, 128, dtype=torch.bfloat16, device=DEV)
    k_l[:, :n, :hd] = k.transpose(0, 1)
    v_pad = torch.zeros(sp, heads, 128, dtype=torch.bfloat16, device=DEV)
    v_pad[:n, :, :hd] = v
    tok = torch.from_numpy(perm16_tokens(sp)).to(DEV)
    vt_l = v_pad[tok].permute(1, 2, 0).contiguous()
    o = torch.full((n, heads * hd), 7.0, dtype=torch.bfloat16, device=DEV)
    nb = b.vision_attention_workspace_bytes(n)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    b.vision_attention(q_l, k_l, vt_l, o, n, heads, hd, grids, 2, ws, nb)
    torch.cuda.synchronize()
    ref = OV.segment_attention(f64(q), f64(k), f64(v), OV.segments(grids))
    r, _, w = report_rows("vision attention", f64(o), ref, hd)
    assert r <= 8e-3 and w <= 3e-2


@pytest.mark.parametrize("vd,grids", [(synth.VISION_TINY, GRIDS_TINY), (synth.VISION_FULL, GRIDS_FULL)])
def test_vision_embed_matches_oracle(vd, grids):
    w, tables, px, n, cfg, ws, nb = _setup(vd, grids)
    h = torch.empty(n, vd.hidden, dtype=torch.bfloat16, device=DEV)
    b.vision_embed(cfg, tables, px, grids, h, ws, nb)
    torch.cuda.synchronize()
    ref = OV.patch_embed(f64(px), f64(w["patch_w"]), f64(w["patch_b"])) + \
        OV.pos_embed_interpolate(f64(w["pos_table"]), grids, vd.pos_side, vd.merge)
    assert report(f"vision embed {vd.hidden}", f64(h), ref)[0] <= 6e-3


# head_dim 128: the per-frame attention's all-dims path (head_dim 72 stops at 96)
VISION_HD128 = synth.VisionDims(hidden=512, n_heads=4, mlp_width=1000, intermediate=1024, depth=2,
                                patch=8, temporal_patch=2, in_channels=3, merge=2, out_hidden=256,
                                pos_side=8, deepstack=(0,))


@pytest.mark.parametrize("vd,grids,blocks", [(synth.VISION_TINY, GRIDS_TINY, [0, 1, 2]),
                                             (synth.VISION_FULL, GRIDS_FULL, [0]),
                                             (VISION_HD128, GRIDS_TINY, [0, 1])])
def test_vision_blocks_teacher_forced(vd, grids, blocks):
    w, tables, px, n, cfg, ws, nb = _setup(vd, grids, seed=1)
    od = _odims(vd)
    g = torch.Generator(device=DEV).manual_seed(3)
    h = torch.randn(n, vd.hidden, generator=g, device=DEV).to(torch.bfloat16)
    ang = OV.rotary_angles(grids, od.head_dim, vd.merge)
    segs = OV.segments(grids)
    for i in blocks:
        h_in = f64(h)
        b.vision_blocks(cfg, tables, i, 1, h, grids, ws, nb)
        torch.cuda.synchronize()
        ref = OV.block(h_in, _oblock(w["blocks"][i], vd.mlp_width), od, ang, segs)
        assert report(f"vision block {i} (hidden {vd.hidden}, teacher-forced)", f64(h), ref)[0] <= 2e-2


def test_vision_frames_are_independent():
    vd, grids = synth.VISION_TINY, GRIDS_TINY
    w, tables, px, n, cfg, ws, nb = _setup(vd, grids, seed=2)
    outs = []
    for bump in (0.0, 1.0):
        p = px.clone()
        p[64:96] += bump                      # first frame of the video only
        h = torch.empty(n, vd.hidden, dtype=torch.bfloat16, device=DEV)
        b.vision_embed(cfg, tables, p, grids, h, ws, nb)
        b.vision_blocks(cfg, tables, 0, vd.depth, h, grids, ws, nb)
        torch.cuda.synchronize()
        outs.append(h.clone())
    same = torch.ones(n, dtype=torch.bool, device=DEV)
    same[64:96] = False
    assert torch.equal(outs[0][same], outs[1][same])
    assert not torch.equal(outs[0][64:96], outs[1][64:96])


@pytest.mark.parametrize("vd", [synth.VISION_TINY, synth.VISION_FULL])
@pytest.mark.parametrize("post", [False, True])
def test_vision_merge_matches_oracle(vd, post):
    n = 512
    w = synth.vision_weights(vd, 3, DEV)
    cfg = b.vision_config(vd)
    nb = b.vision_workspace_bytes(cfg, n)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(4)
    h = torch.randn(n, vd.hidden, generator=g, device=DEV).to(torch.bfloat16)
    m = w["deepstack"][0] if post else w["merger"]
    out = torch.empty(n // vd.merge ** 2, vd.out_hidden, dtype=torch.bfloat16, device=DEV)
    b.vision_merge(cfg, m, post, h, n, out, ws, nb)
    torch.cuda.synchronize()
    ref = OV.merger(f64(h), _omerger(m), _odims(vd), post)
    assert report(f"vision merger post={post} hidden {vd.hidden}", f64(out), ref)[0] <= 1e-2


@pytest.mark.parametrize("vd,grids,depth", [(synth.VISION_TINY, GRIDS_TINY, None)])
def test_vision_forward_free_running(vd, grids, depth):
    w, tables, px, n, cfg, ws, nb = _setup(vd, grids, seed=4)
    nm = n // vd.merge ** 2
    merged = torch.empty(nm, vd.out_hidden, dtype=torch.bfloat16, device=DEV)
    ds = [torch.empty(nm, vd.out_hidden, dtype=torch.bfloat16, device=DEV) for _ in vd.deepstack]
    b.vision_forward(cfg, tables, px, grids, merged, ds, ws, nb)
    torch.cuda.synchronize()
    ow = {"patch_w": f64(w["patch_w"]), "patch_b": f64(w["patch_b"]),
          "pos_table": f64(w["pos_table"]),
          "blocks": [_oblock(p, vd.mlp_width) for p in w["blocks"]],
          "merger": _omerger(w["merger"]), "deepstack": [_omerger(m) for m in w["deepstack"]]}
    out, ref_ds = OV.forward(f64(px), grids, ow, _odims(vd))
    assert report("vision tower merged (free-running)", f64(merged), out)[0] <= 5e-2
    for l, (got, ref) in enumerate(zip(ds, ref_ds)):
        assert report(f"vision tower DeepStack {l}", f64(got), ref)[0] <= 5e-2


def test_vision_forward_full_depth_free_running():
    """The full 27-block, full-width tower with its three DeepStack mergers,
    free-running on an image and a two-frame video."""
    print(f"vision tower full depth, grids {GRIDS_FULL}", flush=True)
    test_vision_forward_free_running(synth.VISION_FULL, GRIDS_FULL, None)


def test_vision_block_benched_grid_teacher_forced():
    """One full-width block on the single 64 x 128-patch frame the bench times
    (8192 patches attending to each other), every output against the oracle."""
    vd, grids = synth.VISION_FULL, [(1, 64, 128)]
    print(f"vision block on the benched grid {grids}", flush=True)
    test_vision_blocks_teacher_forced(vd, grids, [5])


def test_vision_forward_full_width_short_stack():
    # the full-width tower with 4 blocks and DeepStack after blocks 1 and 3
    vd = synth.VisionDims(**{**synth.VISION_FULL.__dict__, "depth": 4, "deepstack": (1, 3)})
    test_vision_forward_free_running(vd, GRIDS_FULL, None)


def test_vision_rejects_bad_grids():
    vd = synth.VISION_TINY
    w, tables, px, n, cfg, ws, nb = _setup(vd, GRIDS_TINY)
    h = torch.empty(n, vd.hidden, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(b.MheError):
        b.vision_embed(cfg, tables, px, [(1, 7, 8)], h, ws, nb)      # h not a multiple of merge
    with pytest.raises(b.MheError):
        b.vision_blocks(cfg, tables, 0, vd.depth + 1, h, GRIDS_TINY, ws, nb)
