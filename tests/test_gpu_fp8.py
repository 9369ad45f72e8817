"""The FP8 (per-tensor E4M3) path through the C ABI against the oracle's FP8
reading (oracle/fp8.py).

Bars, from the arithmetic:
  * quantisation takes the same fp32 factor, product, clamp and
    round-to-nearest-even as the oracle on the same bf16 input, so codes must
    be bit-identical (compared as values, every code decoded by the E4M3
    table) and the scale equal to within one fp32 rounding;
  * the FP8 GEMMs on identical codes and scales differ from the float64 sum
    only by fp32 accumulation and one bf16 rounding: rel-L2 <= 4e-3 as for the
    bf16 GEMMs;
  * a layer: the GPU quantises its bf16 activations, the oracle its float64
    ones, so a code whose input moved (bf16 rounding of the steps before)
    may land one E4M3 step away: the two quantisations round the same tensor
    nearly independently. The layer's update (output - input) may then
    differ from the FP8 oracle's by up to sqrt(2) times the FP8 rounding
    error itself (the oracle's FP8 update against its bf16 update); the bar
    is 1.5 times that, so any error source beyond FP8 rounding (a wrong or
    stale scale, a dropped clamp, a wrong tensor) fails it. The output
    (residual included) meets the bf16 layer's bar, rel-L2 <= 2e-2, or, where
    the FP8 rounding of a large update alone moves the output further (the
    oracle's FP8 output against its bf16 output), 1.5 times that distance:
    in the first layer of the seq-4096 stack the update is as large as the
    output and FP8 rounding moves it by ~6.6e-2.
Inputs are seeded (synth), bf16-valued or random E4M3 codes.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as Q
from multimodal_encoder_prefill_amd import binding as b
from multimodal_encoder_prefill_amd import synth
from helpers import f64, report, rel_l2, oracle_dims, oracle_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"
TABLE = Q.e4m3_values()


def _decode(q: torch.Tensor) -> np.ndarray:
    return TABLE[q.cpu().numpy()]


def _randn(shape, seed, std=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * std).to(torch.bfloat16)


def _qws():
    return torch.empty(b.quantize_fp8_workspace_bytes(), device=DEV, dtype=torch.uint8)


def _gemm_ws():
    return torch.empty(b.linear_workspace_bytes(), device=DEV, dtype=torch.uint8)


# ------------------------------------------------------------------ quantisation

def _wide(shape, seed):
    """Values over ~20 binades (E4M3 subnormals after scaling included)."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    mag = torch.exp2(torch.rand(shape, generator=g, device=DEV) * 20 - 16)
    sign = torch.where(torch.rand(shape, generator=g, device=DEV) < 0.5, -1.0, 1.0)
    return (mag * sign).to(torch.bfloat16)


@pytest.mark.parametrize("case,rows,cols", [
    ("normal", 300, 640), ("wide", 257, 1024), ("outlier", 64, 5120), ("one_row", 1, 8),
    ("tall", 4096, 5120),
])
def test_quantize_bit_exact(case, rows, cols):
    print(f"quantize {case} {rows}x{cols}", flush=True)
    if case == "wide":
        x = _wide((rows, cols), 70)
    else:
        x = _randn((rows, cols), 71 + rows)
    if case == "outlier":
        x[17, 33] = 3000.0
    q = torch.empty((rows, cols), device=DEV, dtype=torch.uint8)
    s = torch.empty(1, device=DEV, dtype=torch.float32)
    b.quantize_fp8([x], [rows], cols, q, s, _qws())
    torch.cuda.synchronize()
    vals, scale = Q.quantize(f64(x))
    got = _decode(q)
    assert not np.any(np.isnan(got))
    mism = np.count_nonzero(got != vals)
    print(f"  code mismatches: {mism} of {got.size}; scale {s.item():.9g} vs {scale:.9g}", flush=True)
    assert mism == 0
    assert abs(s.item() - scale) <= 2.0 ** -23 * scale


def test_quantize_fused_parts_share_one_scale():
    """Three row blocks quantised as one tensor equal the quantisation of their stack."""
    parts = [_randn((r, 512), 80 + i, std) for i, (r, std) in enumerate([(100, 1.0), (37, 5.0), (163, 0.1)])]
    rows = [100, 37, 163]
    q = torch.empty((300, 512), device=DEV, dtype=torch.uint8)
    s = torch.empty(1, device=DEV, dtype=torch.float32)
    b.quantize_fp8(parts, rows, 512, q, s, _qws())
    torch.cuda.synchronize()
    vals, scale = Q.quantize(np.concatenate([f64(p) for p in parts]))
    assert np.array_equal(_decode(q), vals)
    assert abs(s.item() - scale) <= 2.0 ** -23 * scale


def test_quantize_all_zero():
    x = torch.zeros((40, 256), device=DEV, dtype=torch.bfloat16)
    q = torch.full((40, 256), 0x55, device=DEV, dtype=torch.uint8)
    s = torch.zeros(1, device=DEV, dtype=torch.float32)
    b.quantize_fp8([x], [40], 256, q, s, _qws())
    torch.cuda.synchronize()
    assert np.all(_decode(q) == 0.0) and s.item() == 1.0


# ------------------------------------------------------------------ FP8 GEMMs

def _codes(shape, seed):
    return synth.fp8_codes(shape, seed, DEV)


def _scale(v):
    return torch.tensor([v], device=DEV, dtype=torch.float32)


FP8_SHAPES = [(64, 64, 128), (300, 96, 256), (256, 256, 256), (513, 1056, 640), (1000, 2048, 1024)]


@pytest.mark.parametrize("m,n,k", FP8_SHAPES)
@pytest.mark.parametrize("residual", [False, True])
def test_linear_fp8(m, n, k, residual):
    print(f"linear_fp8 m={m} n={n} k={k} residual={residual}", flush=True)
    a, w = _codes((m, k), 1 + m), _codes((n, k), 2 + n)
    sa, sw = _scale(0.0123), _scale(3.1e-3)
    c = _randn((m, n), 30) if residual else torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    r0 = f64(c) if residual else 0.0
    b.linear_fp8(a, sa, w, sw, c, m, n, k, residual=c if residual else None)
    torch.cuda.synchronize()
    ref = r0 + (_decode(a) @ _decode(w).T) * (float(sa.item()) * float(sw.item()))
    r, mx = report("linear_fp8", f64(c), ref)
    assert r <= 4e-3
    assert mx <= 2.0 ** -7 * np.max(np.abs(ref))


@pytest.mark.parametrize("m,n,k", [(64, 64, 128), (300, 96, 256), (513, 1056, 640)])
def test_linear_swiglu_fp8(m, n, k):
    print(f"swiglu_fp8 m={m} n={n} k={k}", flush=True)
    a, wgu = _codes((m, k), 3), _codes((2 * n, k), 4)
    sa, sw = _scale(0.01), _scale(2e-3)
    c = torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    b.linear_swiglu_fp8(a, sa, wgu, sw, c, m, n, k)
    torch.cuda.synchronize()
    prod = (_decode(a) @ _decode(wgu).T) * (float(sa.item()) * float(sw.item()))
    ref = oracle.silu(prod[:, :n]) * prod[:, n:]
    r, mx = report("swiglu_fp8", f64(c), ref)
    assert r <= 4e-3
    assert mx <= 2.0 ** -7 * np.max(np.abs(ref))


@pytest.mark.parametrize("m,n,k,residual", [
    (512, 5120, 8192, True),      # 40 tiles, all split along k
    (300, 96, 1024, False),       # ragged m, partial n tile, split
    (4096, 5120, 25600, True),    # down projection: whole tiles + split last wave
])
def test_linear_fp8_split_k(m, n, k, residual):
    print(f"linear_fp8 split-k m={m} n={n} k={k}", flush=True)
    a, w = _codes((m, k), 5 + m), _codes((n, k), 6 + n)
    sa, sw = _scale(0.002), _scale(4e-4)
    c = _randn((m, n), 14) if residual else torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    r0 = f64(c) if residual else 0.0
    c_plain = c.clone()
    b.linear_fp8(a, sa, w, sw, c, m, n, k, residual=c if residual else None, workspace=_gemm_ws())
    b.linear_fp8(a, sa, w, sw, c_plain, m, n, k, residual=c_plain if residual else None)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, m - 1, 24).astype(int))
    ref = (r0[rows] if residual else 0.0) + (_decode(a[rows]) @ _decode(w).T) * (float(sa.item()) * float(sw.item()))
    assert report("linear_fp8 split-k", f64(c)[rows], ref)[0] <= 4e-3
    r, mx = report("split vs unsplit", f64(c), f64(c_plain))
    assert r <= 2e-3 and mx <= 2.0 ** -6 * np.max(np.abs(f64(c_plain)))


@pytest.mark.parametrize("m,n,k", [
    (512, 1280, 4096),   # 20 tiles, all split along k
    (300, 96, 1024),     # ragged m, partial n tile, split
])
def test_linear_swiglu_fp8_split_k(m, n, k):
    print(f"swiglu_fp8 split-k m={m} n={n} k={k}", flush=True)
    a, wgu = _codes((m, k), 15 + m), _codes((2 * n, k), 16 + n)
    sa, sw = _scale(0.002), _scale(4e-4)
    c = torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    c_plain = torch.empty_like(c)
    b.linear_swiglu_fp8(a, sa, wgu, sw, c, m, n, k, workspace=_gemm_ws())
    b.linear_swiglu_fp8(a, sa, wgu, sw, c_plain, m, n, k)
    torch.cuda.synchronize()
    prod = (_decode(a) @ _decode(wgu).T) * (float(sa.item()) * float(sw.item()))
    ref = oracle.silu(prod[:, :n]) * prod[:, n:]
    r, mx = report("swiglu_fp8 split-k", f64(c), ref)
    assert r <= 4e-3
    assert mx <= 2.0 ** -7 * np.max(np.abs(ref))
    r, mx = report("split vs unsplit", f64(c), f64(c_plain))
    assert r <= 2e-3 and mx <= 2.0 ** -6 * np.max(np.abs(f64(c_plain)))


def test_swiglu_fp8_full_size_sampled_rows():
    m, n, k = 4096, 25600, 5120
    a, wgu = _codes((m, k), 7), _codes((2 * n, k), 8)
    sa, sw = _scale(0.004), _scale(1e-3)
    c = torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    b.linear_swiglu_fp8(a, sa, wgu, sw, c, m, n, k, workspace=_gemm_ws())
    torch.cuda.synchronize()
    rows = np.array([0, 17, 511, 2048, 4095])
    prod = (_decode(a[rows]) @ _decode(wgu).T) * (float(sa.item()) * float(sw.item()))
    ref = oracle.silu(prod[:, :n]) * prod[:, n:]
    assert report("swiglu_fp8 full sampled", f64(c)[rows], ref)[0] <= 4e-3


def test_linear_fp8_qkv_full_size_sampled_rows():
    m, n, k = 4096, 10240, 5120
    a, w = _codes((m, k), 9), _codes((n, k), 10)
    sa, sw = _scale(0.003), _scale(2e-3)
    c = torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    b.linear_fp8(a, sa, w, sw, c, m, n, k, workspace=_gemm_ws())
    torch.cuda.synchronize()
    rows = np.array([0, 255, 256, 3333, 4095])
    ref = (_decode(a[rows]) @ _decode(w).T) * (float(sa.item()) * float(sw.item()))
    assert report("qkv_fp8 full sampled", f64(c)[rows], ref)[0] <= 4e-3


# ------------------------------------------------------------------ FP8 layer / stack

def _setup(wl):
    layers = [synth.layer_weights(wl, l, DEV) for l in range(wl.n_layers)]
    cfg = b.config_from_dims(wl.dims)
    fp8 = [b.Fp8Layer(w, cfg) for w in layers]
    nbytes = b.workspace_bytes_fp8(cfg, wl.seq)
    return dict(layers=layers, fp8=fp8, cfg=cfg, nbytes=nbytes,
                ws=torch.empty(nbytes, device=DEV, dtype=torch.uint8),
                emb=synth.embeddings(wl, DEV), pos_np=synth.positions(wl),
                pos=torch.from_numpy(synth.positions(wl)).to(DEV),
                mask_np=synth.visual_mask(wl), mask=torch.from_numpy(synth.visual_mask(wl)).to(DEV),
                ds=[synth.deepstack_features(wl, i, DEV) for i in range(wl.n_ds)])


def _gpu_states(wl, s):
    h = s["emb"].clone()
    states = [h.clone()]
    for l, f in enumerate(s["fp8"]):
        b.layer_forward_fp8(s["cfg"], f.table, h, s["pos"], wl.seq, s["ws"], s["nbytes"])
        if l < len(s["ds"]) and wl.n_vis > 0:
            b.deepstack_inject(h, wl.seq, wl.dims.hidden, s["mask"], wl.n_vis, s["ds"][l],
                               s["ws"], s["nbytes"])
        states.append(h.clone())
    torch.cuda.synchronize()
    return states


def _check_layers(wl, s, states, layers, threads=1):
    dims = oracle_dims(wl.dims)
    cos, sin = oracle.rope_cos_sin(s["pos_np"], dims.head_dim, dims.rope_theta, dims.mrope_section)
    idx = np.flatnonzero(s["mask_np"])
    for l in layers:
        h_in = f64(states[l])
        w = oracle_layer(s["layers"][l])
        ref8 = Q.decoder_layer_fp8(h_in, w, Q.quantize_layer(w, threads), cos, sin, dims, threads)
        ref16 = oracle.decoder_layer(h_in, w, cos, sin, dims)
        if l < len(s["ds"]) and wl.n_vis > 0:
            add = np.zeros_like(ref8)
            add[idx] = f64(s["ds"][l])[: len(idx)]
            ref8, ref16 = ref8 + add, ref16 + add
        got = f64(states[l + 1])
        r, _ = report(f"{wl.key} fp8 layer {l} (teacher-forced)", got, ref8)
        upd_gpu = rel_l2(got - h_in, ref8 - h_in)
        upd_fp8 = rel_l2(ref8 - h_in, ref16 - h_in)
        print(f"  update: gpu vs fp8 oracle {upd_gpu:.3e}; fp8 vs bf16 oracle {upd_fp8:.3e}", flush=True)
        out_fp8 = rel_l2(ref8, ref16)
        print(f"  output: fp8 vs bf16 oracle {out_fp8:.3e}", flush=True)
        assert r <= max(2e-2, 1.5 * out_fp8)
        assert upd_gpu <= 1.5 * upd_fp8


def test_fp8_layer_tiny_teacher_forced():
    wl = synth.WORKLOADS["tiny"]
    s = _setup(wl)
    _check_layers(wl, s, _gpu_states(wl, s), range(wl.n_layers))


@pytest.mark.parametrize("seq", [1, 33, 129])
def test_fp8_layers_edge_lengths(seq):
    """The FP8 layer (quantised inputs, the attention with the q norm inside
    it emitting the maxima of its output) at a single token, a partial query
    block and one key tile plus one key, head dim 128 with 8 query heads per
    key/value head: every row of two layers against the oracle's FP8 layer."""
    dims = synth.Dims(hidden=1024, n_heads=8, n_kv_heads=1, head_dim=128, intermediate=2048)
    wl = synth.custom_workload(dims, seq, 2, key=f"fp8_edge_{seq}", index=70 + seq % 20)
    print(f"fp8 edge layers seq={seq}", flush=True)
    s = _setup(wl)
    _check_layers(wl, s, _gpu_states(wl, s), range(wl.n_layers))


def test_fp8_weights_match_oracle_quantisation():
    """The load-time quantisation of a layer (fused qkv and gate_up) is the oracle's, bit for bit."""
    wl = synth.WORKLOADS["tiny"]
    w = synth.layer_weights(wl, 0, DEV)
    f = b.Fp8Layer(w, b.config_from_dims(wl.dims))
    ref = Q.quantize_layer(oracle_layer(w))
    for name in ("w_qkv", "w_o", "w_gate_up", "w_down"):
        vals, scale = ref[name]
        assert np.array_equal(_decode(f.tensors[name]), vals), name
        assert abs(f.tensors["s_" + name[2:]].item() - scale) <= 2.0 ** -23 * scale


def test_encode_fp8_equals_layer_calls_and_tracks_oracle():
    dims = synth.Dims(hidden=512, n_heads=8, n_kv_heads=1, head_dim=64, intermediate=1536,
                      rms_eps=1e-6, rope_theta=1e6)
    segs = (("text", 100), ("visual", (1, 8, 16)), ("text", 72))
    wl = synth.custom_workload(dims, 300, 6, segs, 3, key="narrow_fp8", index=51)
    s = _setup(wl)
    out = torch.empty_like(s["emb"])
    b.encode_fp8(s["cfg"], [f.table for f in s["fp8"]], s["emb"], s["pos"], wl.seq, out, s["ws"],
                 s["nbytes"], visual_mask=s["mask"], n_vis=wl.n_vis, deepstack=s["ds"])
    torch.cuda.synchronize()
    states = _gpu_states(wl, s)
    assert torch.equal(states[-1], out)
    _check_layers(wl, s, states, [0, 2, 5])


_FULL = {}


@pytest.mark.parametrize("layer", [0, 49])
def test_fp8_layer_full_width_s4096_teacher_forced(layer):
    """The FP8 layer at full width in the seq-4096 image stack (the FP8
    encode's own bf16 input of that layer, every row): layer 0 carries
    DeepStack level 0, layer 49 is the last."""
    import os
    if not _FULL:
        wl = synth.WORKLOADS["image_s4096_l50"]
        print(f"fp8 full stack {wl.key}: seq {wl.seq}, {wl.n_layers} layers", flush=True)
        s = _setup(wl)
        _FULL.update(wl=wl, s=s, states=_gpu_states(wl, s))
    wl, s, states = _FULL["wl"], _FULL["s"], _FULL["states"]
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    _check_layers(wl, s, states, [layer], threads)
    if layer == 49:
        _FULL.clear()
        torch.cuda.empty_cache()
