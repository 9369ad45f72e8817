"""Decoder layer and whole-prefill parity of the HIP path against the CPU oracle.

Bars (fixed by the decoder's own accuracy target): one layer, fed the GPU's
bf16 hidden state (teacher-forced), agrees with the float64 oracle to
rel-L2 <= 2e-2; the free-running stack agrees at its last layer to
rel-L2 <= 5e-2. Max-abs is printed beside every rel-L2.

The 50-layer seq-4096 stack is checked free-running on a prefix: attention is
causal and every other step acts on one row, so rows [0, P) of every hidden
state depend on tokens [0, P) only, and the oracle run on the first P tokens
(with their positions, mask and DeepStack rows) gives exactly those rows of
the full stack's output.
"""

import numpy as np
import pytest
import torch

import oracle
from multimodal_encoder_prefill_amd import binding as b
from multimodal_encoder_prefill_amd import synth
from helpers import f64, report, oracle_dims, oracle_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _setup(wl, n_layers=None):
    n_layers = wl.n_layers if n_layers is None else n_layers
    layers = [synth.layer_weights(wl, l, DEV) for l in range(n_layers)]
    emb = synth.embeddings(wl, DEV)
    pos_np = synth.positions(wl)
    pos = torch.from_numpy(pos_np).to(DEV)
    mask_np = synth.visual_mask(wl)
    mask = torch.from_numpy(mask_np).to(DEV)
    ds = [synth.deepstack_features(wl, i, DEV) for i in range(wl.n_ds)]
    cfg = b.config_from_dims(wl.dims)
    nbytes = b.workspace_bytes(cfg, wl.seq)
    ws = torch.empty(nbytes, device=DEV, dtype=torch.uint8)
    return dict(layers=layers, emb=emb, pos=pos, pos_np=pos_np, mask=mask, mask_np=mask_np,
                ds=ds, cfg=cfg, ws=ws, nbytes=nbytes)


def _gpu_states(wl, s):
    """hidden_states[0..L] from the GPU, one layer (and DeepStack level) per call."""
    h = s["emb"].clone()
    states = [h.clone()]
    for l, w in enumerate(s["layers"]):
        b.layer_forward(s["cfg"], w, h, s["pos"], wl.seq, s["ws"], s["nbytes"])
        if l < len(s["ds"]) and wl.n_vis > 0:
            b.deepstack_inject(h, wl.seq, wl.dims.hidden, s["mask"], wl.n_vis, s["ds"][l],
                               s["ws"], s["nbytes"])
        states.append(h.clone())
    torch.cuda.synchronize()
    return states


def _teacher_forced(wl, s, states, rows=None, layers=None):
    dims = oracle_dims(wl.dims)
    cos, sin = oracle.rope_cos_sin(s["pos_np"], dims.head_dim, dims.rope_theta, dims.mrope_section)
    idx = np.flatnonzero(s["mask_np"])
    worst = 0.0
    for l in (range(len(s["layers"])) if layers is None else layers):
        h_in = f64(states[l])
        r = np.arange(wl.seq) if rows is None else rows
        ref = oracle.decoder_layer(h_in, oracle_layer(s["layers"][l]), cos, sin, dims, rows=r)
        if l < len(s["ds"]) and wl.n_vis > 0:
            feat = f64(s["ds"][l])
            pos_in_vis = np.searchsorted(idx, r)
            is_vis = s["mask_np"][r] != 0
            ref[is_vis] += feat[pos_in_vis[is_vis]]
        got = f64(states[l + 1])[r]
        rel, _ = report(f"{wl.key} layer {l} (teacher-forced)", got, ref)
        worst = max(worst, rel)
    return worst


def test_layer_tiny_teacher_forced():
    wl = synth.WORKLOADS["tiny"]
    s = _setup(wl)
    states = _gpu_states(wl, s)
    assert _teacher_forced(wl, s, states) <= 2e-2


def test_layer_full_width_s512_teacher_forced():
    wl = synth.WORKLOADS["layer1_s512"]
    s = _setup(wl)
    states = _gpu_states(wl, s)
    rows = np.unique(np.concatenate([np.arange(0, 512, 17), [1, 255, 256, 510, 511]]))
    assert _teacher_forced(wl, s, states, rows=rows) <= 2e-2


def test_layers_full_width_ragged_seq_every_row():
    """Two full-width layers at a ragged length (seq 777: partial 256-row
    GEMM tiles, the 256-wide tile and its split-K tail instead of the 320-wide
    one, a partial attention tile) with an image block and its DeepStack
    levels: every row of both layers teacher-forced against the oracle."""
    wl = synth.custom_workload(synth.FULL, 777, 2, (("text", 201), ("visual", (1, 16, 32)), ("text", 64)),
                               2, key="full_s777", index=77)
    print(f"full-width layers at seq {wl.seq}, {wl.n_vis} visual tokens", flush=True)
    s = _setup(wl)
    out = _run_encode(wl, s)
    states = _gpu_states(wl, s)
    assert torch.equal(states[-1], out)
    assert _teacher_forced(wl, s, states) <= 2e-2


_EDGE_DIMS = {
    "d128_g8": synth.Dims(hidden=1024, n_heads=8, n_kv_heads=1, head_dim=128, intermediate=2048),
    "d64_g2": synth.Dims(hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=1024,
                         rope_theta=1e6),
}


@pytest.mark.parametrize("seq", [1, 2, 31, 33, 127, 129, 255])
@pytest.mark.parametrize("key", sorted(_EDGE_DIMS))
def test_layers_edge_lengths_every_row(key, seq):
    """Two layers at lengths around the 32-query block and the 128-key tile
    (one token, a partial query block, one key tile plus one key): the layer
    path's q norm and rotary inside the attention, the k-only norm kernel and
    the padded K / V^T layouts, every row teacher-forced against the oracle;
    mhe_encode equals the layer-by-layer calls."""
    wl = synth.custom_workload(_EDGE_DIMS[key], seq, 2, key=f"edge_{key}_{seq}", index=60 + seq % 30)
    print(f"edge layers {key} seq={seq}", flush=True)
    s = _setup(wl)
    out = _run_encode(wl, s)
    states = _gpu_states(wl, s)
    assert torch.equal(states[-1], out)
    assert _teacher_forced(wl, s, states) <= 2e-2


def _run_encode(wl, s, n_layers=None):
    layers = s["layers"] if n_layers is None else s["layers"][:n_layers]
    out = torch.empty_like(s["emb"])
    b.encode(s["cfg"], layers, s["emb"], s["pos"], wl.seq, out, s["ws"], s["nbytes"],
             visual_mask=s["mask"] if wl.n_vis else None, n_vis=wl.n_vis,
             deepstack=s["ds"] if wl.n_vis else None)
    torch.cuda.synchronize()
    return out


def test_encode_tiny_free_running():
    wl = synth.WORKLOADS["tiny"]
    s = _setup(wl)
    emb0 = s["emb"].clone()
    out = _run_encode(wl, s)
    assert torch.equal(s["emb"], emb0)                       # input not written
    ref = oracle.encode(f64(s["emb"]), s["pos_np"], [oracle_layer(w) for w in s["layers"]],
                        oracle_dims(wl.dims))
    assert report("tiny layer-2 free-running", f64(out), ref)[0] <= 5e-2


def _narrow_stack(n_layers, seq, grid, n_ds):
    dims = synth.Dims(hidden=512, n_heads=8, n_kv_heads=1, head_dim=64, intermediate=1536,
                      rms_eps=1e-6, rope_theta=1e6)
    text = (seq - int(np.prod(grid))) // 2
    segs = (("text", text), ("visual", grid), ("text", seq - text - int(np.prod(grid))))
    return synth.custom_workload(dims, seq, n_layers, segs, n_ds, key="narrow50", index=50)


def test_encode_50_layers_narrow_free_running():
    """50 layers free-running, every DeepStack level, image segment: the error at
    hidden_states[50] stays within the end-to-end bar."""
    wl = _narrow_stack(50, 300, (1, 8, 16), 3)
    s = _setup(wl)
    out = _run_encode(wl, s)
    states = oracle.encode(f64(s["emb"]), s["pos_np"], [oracle_layer(w) for w in s["layers"]],
                           oracle_dims(wl.dims), visual_mask=s["mask_np"],
                           deepstack=[f64(d) for d in s["ds"]], return_all=True)
    assert report("narrow hidden_states[50] free-running", f64(out), states[-1])[0] <= 5e-2
    gpu_states = _gpu_states(wl, s)
    assert torch.equal(gpu_states[-1], out)                  # encode == layer-by-layer calls
    assert _teacher_forced(wl, s, gpu_states, layers=[0, 1, 2, 3, 25, 49]) <= 2e-2


class _OracleWalk:
    """The oracle walked layer by layer beside the GPU's per-layer states:
    free-running on the first `prefix` tokens, and teacher-forced (the GPU's
    bf16 input of each layer) on the rows `tf_rows`. Each layer's weights are
    converted to float64 once and serve both."""

    def __init__(self, wl, s, prefix, tf_rows):
        self.wl, self.s, self.P = wl, s, prefix
        self.dims = oracle_dims(wl.dims)
        self.cos, self.sin = oracle.rope_cos_sin(s["pos_np"], self.dims.head_dim,
                                                 self.dims.rope_theta, self.dims.mrope_section)
        self.idx = np.flatnonzero(s["mask_np"])
        self.h = f64(s["emb"][:prefix])
        self.tf_rows = np.asarray(tf_rows)
        self.done = 0
        self.log = []       # per layer: (teacher-forced rel, max-abs, free-running rel, max-abs)

    def _ds(self, l, rows):
        """DeepStack level l's rows for the tokens `rows` (zero off the visual tokens)."""
        add = np.zeros((len(rows), self.wl.dims.hidden))
        if l < len(self.s["ds"]) and self.wl.n_vis > 0:
            is_vis = self.s["mask_np"][rows] != 0
            add[is_vis] = f64(self.s["ds"][l])[np.searchsorted(self.idx, rows[is_vis])]
        return add

    def advance(self, states, upto):
        for l in range(self.done, upto):
            w = oracle_layer(self.s["layers"][l])
            pre = np.arange(self.P)
            self.h = oracle.decoder_layer(self.h, w, self.cos, self.sin, self.dims) + self._ds(l, pre)
            fr, fm = report(f"{self.wl.key} rows [0, {self.P}) after layer {l} (free-running)",
                            f64(states[l + 1][:self.P]), self.h)
            r = self.tf_rows
            ref = oracle.decoder_layer(f64(states[l]), w, self.cos, self.sin, self.dims, rows=r)
            tr, tm = report(f"{self.wl.key} layer {l} on {len(r)} rows (teacher-forced)",
                            f64(states[l + 1])[r], ref + self._ds(l, r))
            self.log.append((tr, tm, fr, fm))
            self.done = l + 1


def test_encode_image_s2048_l4_every_row():
    """Four full-width layers, seq 2048 with a 1x32x32 image and its DeepStack
    levels: every row of every layer teacher-forced, and the free-running
    output, against the oracle; mhe_encode equals the layer-by-layer calls."""
    wl = synth.WORKLOADS["image_s2048_l4"]
    s = _setup(wl)
    out = _run_encode(wl, s)
    states = _gpu_states(wl, s)
    assert torch.equal(states[-1], out)
    walk = _OracleWalk(wl, s, wl.seq, np.arange(wl.seq))
    walk.advance(states, wl.n_layers)
    assert max(t[0] for t in walk.log) <= 2e-2
    assert walk.log[-1][2] <= 5e-2


# The 50-layer seq-4096 image stack, in the launch configuration bench.py
# times. P = 1152: the 1024 leading text tokens and the first two rows (128
# tokens) of the 1x32x64 image block, which carry all three DeepStack levels
# and distinct T/H/W positions. Teacher-forced rows: every 32nd row of the
# prefix, the image block's edges and an even spread over the whole sequence.
FULL_PREFIX = 1152
_FULL = {}


def _full_stack():
    if "walk" not in _FULL:
        wl = synth.WORKLOADS["image_s4096_l50"]
        print(f"full stack {wl.key}: seq {wl.seq}, {wl.n_layers} layers, prefix {FULL_PREFIX}", flush=True)
        s = _setup(wl)
        out = _run_encode(wl, s)
        states = _gpu_states(wl, s)
        assert torch.equal(states[-1], out)
        vis = np.flatnonzero(s["mask_np"])
        rows = np.unique(np.concatenate([
            np.arange(0, FULL_PREFIX, 32), [0, 1, vis[0] - 1, vis[0], vis[0] + 63, vis[0] + 64,
                                             vis[-1], vis[-1] + 1, wl.seq - 1],
            np.linspace(0, wl.seq - 1, 17).astype(int)]))
        _FULL.update(wl=wl, s=s, out=out, states=states,
                     walk=_OracleWalk(wl, s, FULL_PREFIX, rows))
    return _FULL


@pytest.mark.parametrize("chunk", range(5))
def test_encode_image_s4096_l50_layers(chunk):
    """Layers [10 chunk, 10 chunk + 10) of the 50-layer stack: teacher-forced
    on the sampled rows (<= 2e-2 each), free-running on the prefix; the last
    chunk checks hidden_states[50] free-running (<= 5e-2) on the prefix."""
    f = _full_stack()
    walk = f["walk"]
    lo, hi = 10 * chunk, 10 * chunk + 10
    walk.advance(f["states"], hi)
    assert max(t[0] for t in walk.log[lo:hi]) <= 2e-2
    if hi == f["wl"].n_layers:
        rel, mx = report("image_s4096_l50 hidden_states[50] rows [0, 1152) (free-running)",
                         f64(f["out"][:FULL_PREFIX]), walk.h)
        worst = max(walk.log, key=lambda t: t[0])
        print(f"worst teacher-forced layer: rel_l2={worst[0]:.3e} max_abs={worst[1]:.3e}", flush=True)
        _FULL.clear()
        torch.cuda.empty_cache()
        assert rel <= 5e-2


def test_encode_causal_bitwise():
    wl = _narrow_stack(3, 200, (1, 4, 8), 2)
    s = _setup(wl)
    out1 = _run_encode(wl, s)
    cut = 120
    s["emb"][cut:] += 1.0
    out2 = _run_encode(wl, s)
    assert torch.equal(out1[:cut], out2[:cut])
    assert not torch.equal(out1[cut:], out2[cut:])


def test_encode_no_deepstack_when_no_visual_tokens():
    wl = synth.WORKLOADS["tiny"]
    s = _setup(wl)
    out = _run_encode(wl, s)
    out2 = torch.empty_like(out)
    b.encode(s["cfg"], s["layers"], s["emb"], s["pos"], wl.seq, out2, s["ws"], s["nbytes"],
             visual_mask=None, n_vis=0, deepstack=None)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


# The 50-layer seq-16384 video stack: free-running on a prefix of P = 1088
# tokens (the 1024 leading text tokens and the first two rows of the first
# frame, which carry all three DeepStack levels), teacher-forced on every
# layer at rows sampled over the whole sequence (the video block's edges,
# both ends, an even spread). Five chunks of 10 layers, as for the image stack.
VIDEO_PREFIX = 1088
_VIDEO = {}


def _video_stack():
    if "walk" not in _VIDEO:
        wl = synth.WORKLOADS["video_s16384_l50"]
        print(f"full stack {wl.key}: seq {wl.seq}, {wl.n_layers} layers, {wl.n_vis} visual tokens, "
              f"prefix {VIDEO_PREFIX}", flush=True)
        s = _setup(wl)
        out = _run_encode(wl, s)
        states = _gpu_states(wl, s)
        assert torch.equal(states[-1], out)                  # encode == layer-by-layer calls
        vis = np.flatnonzero(s["mask_np"])
        rows = np.unique(np.concatenate([[0, 1, vis[0] - 1, vis[0], vis[-1], vis[-1] + 1, wl.seq - 1],
                                         np.linspace(0, wl.seq - 1, 9).astype(int)]))
        _VIDEO.update(wl=wl, s=s, out=out, states=states,
                      walk=_OracleWalk(wl, s, VIDEO_PREFIX, rows))
    return _VIDEO


@pytest.mark.parametrize("chunk", range(5))
def test_encode_video_s16384_l50_layers(chunk):
    """Layers [10 chunk, 10 chunk + 10) of the 50-layer video stack:
    teacher-forced on the sampled rows (<= 2e-2 each), free-running on the
    prefix; the last chunk checks hidden_states[50] on the prefix (<= 5e-2)."""
    f = _video_stack()
    walk = f["walk"]
    lo, hi = 10 * chunk, 10 * chunk + 10
    walk.advance(f["states"], hi)
    assert max(t[0] for t in walk.log[lo:hi]) <= 2e-2
    if hi == f["wl"].n_layers:
        rel, mx = report(f"video_s16384_l50 hidden_states[50] rows [0, {VIDEO_PREFIX}) (free-running)",
                         f64(f["out"][:VIDEO_PREFIX]), walk.h)
        worst = max(walk.log, key=lambda t: t[0])
        print(f"worst teacher-forced layer: rel_l2={worst[0]:.3e} max_abs={worst[1]:.3e}", flush=True)
        _VIDEO.clear()
        torch.cuda.empty_cache()
        assert rel <= 5e-2
