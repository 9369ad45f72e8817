"""Property tests over random small shapes (hypothesis): the RMSNorm, q/k norm
+ rotary, attention, DeepStack, GEMM, FP8 and vision-tower kernels, through the C ABI, against the
CPU oracle on shapes drawn at random — ragged sequence lengths and GEMM
shapes, head groupings, head dims, position ranges, rotary sections, input
scales, mask densities, with and without the split-K scratch.

The draws are derandomised (the same cases on every run) and each case prints
its shape before its kernel runs. Bars are those of the per-step tests: one
bf16 rounding of each output (rel-L2 <= 4e-3; attention, which also rounds
the probabilities, 8e-3) and, per (token, head) row, <= 3e-2.
"""

import dataclasses

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from multimodal_encoder_prefill_amd import binding as b
from multimodal_encoder_prefill_amd import synth
from helpers import f64, perm16_tokens, report, report_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
ROW_BAR = 3e-2

CASES = settings(max_examples=12, deadline=None, derandomize=True, database=None,
                 suppress_health_check=list(HealthCheck))


def _randn(shape, seed, std=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * std).to(torch.bfloat16)


def _gain(n, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.rand(n, generator=g, device=DEV) + 0.5).to(torch.bfloat16)


# log-uniform input scales: tiny, unit and large activations
scales = st.sampled_from([1e-2, 0.3, 1.0, 4.0, 60.0])


@CASES
@given(rows=st.integers(1, 300), dim8=st.integers(1, 800), std=scales,
       eps=st.sampled_from([1e-6, 1e-5]), seed=st.integers(0, 2**20))
def test_rms_norm_random_shapes(rows, dim8, std, eps, seed):
    dim = 8 * dim8
    print(f"rms_norm rows={rows} dim={dim} std={std} eps={eps} seed={seed}", flush=True)
    x = _randn((rows, dim), seed, std)
    gamma = _gain(dim, seed + 1)
    y = torch.empty_like(x)
    b.rms_norm(x, gamma, y, rows, dim, eps)
    torch.cuda.synchronize()
    ref = oracle.rms_norm(f64(x), f64(gamma), eps)
    assert report("rms_norm", f64(y), ref)[0] <= 4e-3
    assert np.all(np.abs(f64(y) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


@st.composite
def qk_shapes(draw):
    d = draw(st.sampled_from([64, 128]))
    n_kv = draw(st.sampled_from([1, 2, 4, 8]))
    group = draw(st.sampled_from([1, 2, 4, 8]))
    seq = draw(st.integers(1, 300))
    # rotary sections covering the D/2 slots in some split
    a = draw(st.integers(0, d // 2))
    c = draw(st.integers(0, d // 2 - a))
    section = (d // 2 - a - c, a, c)
    theta = draw(st.sampled_from([1e4, 1e6, 5e6]))
    max_pos = draw(st.sampled_from([1, 50, 3000, 16384]))
    return d, n_kv, group, seq, section, theta, max_pos


@CASES
@given(shape=qk_shapes(), seed=st.integers(0, 2**20))
def test_qk_norm_rope_random_shapes(shape, seed):
    d, n_kv, group, seq, section, theta, max_pos = shape
    print(f"qk_norm_rope D={d} heads={n_kv * group}/{n_kv} seq={seq} section={section} "
          f"theta={theta} max_pos={max_pos} seed={seed}", flush=True)
    dims = dataclasses.replace(synth.TINY, hidden=n_kv * group * d, n_heads=n_kv * group,
                               n_kv_heads=n_kv, head_dim=d, rope_theta=theta,
                               mrope_section=section)
    qw, kvw = dims.q_width, dims.kv_width
    qkv = _randn((seq, qw + 2 * kvw), seed, 2.0)
    qn, kn = _gain(d, seed + 1), _gain(d, seed + 2)
    sp = b.seq_pad(seq)
    q_out = torch.full((seq, dims.n_heads, d), 7.0, device=DEV, dtype=torch.bfloat16)
    k_out = torch.full((n_kv, sp, d), 7.0, device=DEV, dtype=torch.bfloat16)
    vt_out = torch.full((n_kv, d, sp), 7.0, device=DEV, dtype=torch.bfloat16)
    positions = synth.random_positions(seq, max_pos, seed=seed)
    pos = torch.from_numpy(np.ascontiguousarray(positions)).to(DEV)
    b.qk_norm_rope(b.config_from_dims(dims), qkv, qn, kn, pos, seq, q_out, k_out, vt_out)
    torch.cuda.synchronize()
    x = f64(qkv)
    cos, sin = oracle.rope_cos_sin(positions, d, theta, section)
    q_ref = oracle.apply_rope(oracle.rms_norm(x[:, :qw].reshape(seq, -1, d), f64(qn), dims.rms_eps), cos, sin)
    k_ref = oracle.apply_rope(oracle.rms_norm(x[:, qw:qw + kvw].reshape(seq, -1, d), f64(kn), dims.rms_eps),
                              cos, sin)
    r, _, w = report_rows("q", f64(q_out), q_ref, d)
    assert r <= 4e-3 and w <= ROW_BAR
    kk = f64(k_out)
    r, _, w = report_rows("k", kk[:, :seq].transpose(1, 0, 2), k_ref, d)
    assert r <= 4e-3 and w <= ROW_BAR
    assert np.all(kk[:, seq:] == 0)
    v_pad = np.zeros((sp, n_kv, d))
    v_pad[:seq] = x[:, qw + kvw:].reshape(seq, n_kv, d)
    assert np.array_equal(f64(vt_out), v_pad[perm16_tokens(sp)].transpose(1, 2, 0))


@CASES
@given(shape=qk_shapes(), seed=st.integers(0, 2**20))
def test_qnorm_attention_random_shapes(shape, seed):
    """The decoder layer's attention step (q RMSNorm and rotary applied as the
    attention kernel loads the raw q rows) on the same random shapes, rotary
    sections and positions, against the oracle's norm, rotary and attention."""
    d, n_kv, group, seq, section, theta, max_pos = shape
    print(f"qnorm_attention D={d} heads={n_kv * group}/{n_kv} seq={seq} section={section} "
          f"theta={theta} max_pos={max_pos} seed={seed}", flush=True)
    dims = dataclasses.replace(synth.TINY, hidden=n_kv * group * d, n_heads=n_kv * group,
                               n_kv_heads=n_kv, head_dim=d, rope_theta=theta,
                               mrope_section=section)
    qw, kvw = dims.q_width, dims.kv_width
    qkv = _randn((seq, qw + 2 * kvw), seed, 2.0)
    qn, kn = _gain(d, seed + 1), _gain(d, seed + 2)
    sp = b.seq_pad(seq)
    q_out = torch.empty((seq, dims.n_heads, d), device=DEV, dtype=torch.bfloat16)
    k_out = torch.empty((n_kv, sp, d), device=DEV, dtype=torch.bfloat16)
    vt_out = torch.empty((n_kv, d, sp), device=DEV, dtype=torch.bfloat16)
    positions = synth.random_positions(seq, max_pos, seed=seed)
    pos = torch.from_numpy(np.ascontiguousarray(positions)).to(DEV)
    cfg = b.config_from_dims(dims)
    b.qk_norm_rope(cfg, qkv, qn, kn, pos, seq, q_out, k_out, vt_out)
    nbytes = b.qnorm_attention_workspace_bytes(cfg, seq)
    ws = torch.empty(nbytes, device=DEV, dtype=torch.uint8)
    o = torch.full((seq, dims.n_heads * d), 7.0, device=DEV, dtype=torch.bfloat16)
    b.qnorm_attention(cfg, qkv, qn, pos, k_out, vt_out, o, seq, ws, nbytes)
    torch.cuda.synchronize()
    x = f64(qkv)
    cos, sin = oracle.rope_cos_sin(positions, d, theta, section)
    q_ref = oracle.apply_rope(oracle.rms_norm(x[:, :qw].reshape(seq, -1, d), f64(qn), dims.rms_eps), cos, sin)
    k_ref = oracle.apply_rope(oracle.rms_norm(x[:, qw:qw + kvw].reshape(seq, -1, d), f64(kn), dims.rms_eps),
                              cos, sin)
    ref = oracle.causal_gqa_attention(q_ref, k_ref, x[:, qw + kvw:].reshape(seq, n_kv, d))
    r, _, w = report_rows("qnorm attention", f64(o), ref.reshape(seq, -1), d)
    assert r <= 8e-3 and w <= ROW_BAR


@st.composite
def attention_shapes(draw):
    d = draw(st.sampled_from([64, 128]))
    n_kv = draw(st.sampled_from([1, 2, 4, 8]))
    group = draw(st.sampled_from([1, 2, 4, 8]))
    seq = draw(st.integers(1, 400))
    return d, n_kv, group, seq


@CASES
@given(shape=attention_shapes(), std=st.sampled_from([0.3, 1.0, 2.0, 4.0]), seed=st.integers(0, 2**20))
def test_attention_random_shapes(shape, std, seed):
    d, n_kv, group, seq = shape
    hq = n_kv * group
    print(f"attention D={d} heads={hq}/{n_kv} seq={seq} std={std} seed={seed}", flush=True)
    q = _randn((seq, hq, d), seed, std)
    k = _randn((seq, n_kv, d), seed + 1, std)
    v = _randn((seq, n_kv, d), seed + 2)
    sp = b.seq_pad(seq)
    k_l = torch.zeros((n_kv, sp, d), device=DEV, dtype=torch.bfloat16)
    k_l[:, :seq] = k.transpose(0, 1)
    v_pad = torch.zeros((sp, n_kv, d), device=DEV, dtype=torch.bfloat16)
    v_pad[:seq] = v
    vt_l = v_pad[torch.from_numpy(perm16_tokens(sp)).to(DEV)].permute(1, 2, 0).contiguous()
    o = torch.full((seq, hq * d), 7.0, device=DEV, dtype=torch.bfloat16)
    b.attention(q, k_l, vt_l, o, seq, hq, n_kv, d)
    torch.cuda.synchronize()
    ref = oracle.causal_gqa_attention(f64(q), f64(k), f64(v)).reshape(seq, hq * d)
    r, _, w = report_rows("attention", f64(o), ref, d)
    assert r <= 8e-3 and w <= ROW_BAR


@CASES
@given(seq=st.integers(1, 2000), dim8=st.integers(1, 700), density=st.floats(0.0, 1.0),
       seed=st.integers(0, 2**20))
def test_deepstack_random_masks(seq, dim8, density, seed):
    dim = 8 * dim8
    print(f"deepstack seq={seq} dim={dim} density={density:.3f} seed={seed}", flush=True)
    rng = np.random.default_rng(seed)
    mask = (rng.random(seq) < density).astype(np.uint8)
    n_vis = int(mask.sum())
    h = _randn((seq, dim), seed)
    feat = _randn((max(n_vis, 1), dim), seed + 1)
    ref = oracle.deepstack_add(f64(h), mask, f64(feat)[:n_vis])
    ws = torch.empty(seq * 4 + 512, device=DEV, dtype=torch.uint8)
    m = torch.from_numpy(mask).to(DEV)
    b.deepstack_inject(h, seq, dim, m, n_vis, feat, ws, ws.numel())
    torch.cuda.synchronize()
    got = f64(h)
    # one rounding of the exact sum of two bf16 values: within half an ulp
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref))
    assert np.array_equal(got[mask == 0], ref[mask == 0])


@st.composite
def gemm_shapes(draw):
    m = draw(st.integers(1, 1100))
    n = 32 * draw(st.integers(1, 64))
    k = 64 * draw(st.integers(1, 32))
    return m, n, k


@CASES
@given(shape=gemm_shapes(), residual=st.booleans(), split=st.booleans(), std=st.sampled_from([0.1, 1.0, 8.0]),
       seed=st.integers(0, 2**20))
def test_linear_random_shapes(shape, residual, split, std, seed):
    """C = A W^T (+ R) on ragged shapes; with the scratch, the last wave may be split along k."""
    m, n, k = shape
    print(f"linear m={m} n={n} k={k} residual={residual} split={split} std={std} seed={seed}", flush=True)
    a = _randn((m, k), seed, std)
    w = _randn((n, k), seed + 1, 0.05)
    c = _randn((m, n), seed + 2) if residual else torch.full((m, n), 7.0, device=DEV, dtype=torch.bfloat16)
    r0 = f64(c) if residual else 0.0
    ws = torch.empty(b.linear_workspace_bytes(), device=DEV, dtype=torch.uint8) if split else None
    b.linear(a, w, c, m, n, k, residual=c if residual else None, workspace=ws)
    torch.cuda.synchronize()
    ref = r0 + f64(a) @ f64(w).T
    r, mx = report("linear", f64(c), ref)
    assert r <= 4e-3
    assert mx <= 2.0 ** -7 * np.max(np.abs(ref))


@CASES
@given(shape=gemm_shapes(), split=st.booleans(), seed=st.integers(0, 2**20))
def test_swiglu_random_shapes(shape, split, seed):
    """silu(A Wg^T) * (A Wu^T) on ragged shapes, with and without the split-K scratch."""
    m, n, k = shape
    print(f"swiglu m={m} n={n} k={k} split={split} seed={seed}", flush=True)
    a = _randn((m, k), seed)
    wg = _randn((n, k), seed + 1, 0.1)
    wu = _randn((n, k), seed + 2, 0.1)
    c = torch.full((m, n), 7.0, device=DEV, dtype=torch.bfloat16)
    ws = torch.empty(b.linear_workspace_bytes(), device=DEV, dtype=torch.uint8) if split else None
    b.linear_swiglu(a, wg, wu, c, m, n, k, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.silu(f64(a) @ f64(wg).T) * (f64(a) @ f64(wu).T)
    r, mx = report("swiglu", f64(c), ref)
    assert r <= 4e-3
    assert mx <= 2.0 ** -7 * np.max(np.abs(ref))


# ------------------------------------------------------------------ FP8 (online E4M3)

@CASES
@given(rows=st.integers(1, 700), cols8=st.integers(1, 200), log_std=st.floats(-6, 6),
       n_parts=st.integers(1, 3), outlier=st.booleans(), seed=st.integers(0, 2**20))
def test_quantize_fp8_random_shapes_bit_exact(rows, cols8, log_std, n_parts, outlier, seed):
    """Per-tensor E4M3 codes of 1-3 stacked row blocks at random scales: the
    same fp32 factor, product, clamp and rounding as the oracle, so the codes
    are bit-identical and the scale equal within one fp32 rounding."""
    from oracle import fp8 as Q
    cols = 8 * cols8
    print(f"quantize_fp8 rows={rows} cols={cols} std=2^{log_std:.2f} parts={n_parts} outlier={outlier} "
          f"seed={seed}", flush=True)
    x = _randn((rows, cols), seed, float(2.0 ** log_std))
    if outlier:
        x[rows // 2, cols // 3] = float(2.0 ** (log_std + 9))
    cuts = sorted(set([0, rows] + [int(v) for v in np.random.default_rng(seed).integers(1, rows + 1, n_parts - 1)]))
    parts = [x[a:b_].contiguous() for a, b_ in zip(cuts, cuts[1:]) if b_ > a]
    q = torch.empty((rows, cols), device=DEV, dtype=torch.uint8)
    s = torch.empty(1, device=DEV, dtype=torch.float32)
    ws = torch.empty(b.quantize_fp8_workspace_bytes(), device=DEV, dtype=torch.uint8)
    b.quantize_fp8(parts, [p.shape[0] for p in parts], cols, q, s, ws)
    torch.cuda.synchronize()
    vals, scale = Q.quantize(f64(x))
    got = Q.e4m3_values()[q.cpu().numpy()]
    assert np.count_nonzero(got != vals) == 0
    assert abs(s.item() - scale) <= 2.0 ** -23 * scale


@CASES
@given(m=st.integers(1, 1100), n32=st.integers(1, 64), k128=st.integers(1, 16), residual=st.booleans(),
       split=st.booleans(), seed=st.integers(0, 2**20))
def test_linear_fp8_random_shapes(m, n32, k128, residual, split, seed):
    """(q_a q_w^T) s_a s_w (+ R) on random E4M3 codes and ragged shapes."""
    from oracle import fp8 as Q
    n, k = 32 * n32, 128 * k128
    print(f"linear_fp8 m={m} n={n} k={k} residual={residual} split={split} seed={seed}", flush=True)
    a, w = synth.fp8_codes((m, k), seed, DEV), synth.fp8_codes((n, k), seed + 1, DEV)
    sa = torch.tensor([0.01 * (1 + seed % 7)], device=DEV, dtype=torch.float32)
    sw = torch.tensor([1e-3 * (1 + seed % 5)], device=DEV, dtype=torch.float32)
    c = _randn((m, n), seed + 2) if residual else torch.full((m, n), 7.0, device=DEV, dtype=torch.bfloat16)
    r0 = f64(c) if residual else 0.0
    ws = torch.empty(b.linear_workspace_bytes(), device=DEV, dtype=torch.uint8) if split else None
    b.linear_fp8(a, sa, w, sw, c, m, n, k, residual=c if residual else None, workspace=ws)
    torch.cuda.synchronize()
    T = Q.e4m3_values()
    ref = r0 + (T[a.cpu().numpy()] @ T[w.cpu().numpy()].T) * (float(sa.item()) * float(sw.item()))
    r, mx = report("linear_fp8", f64(c), ref)
    assert r <= 4e-3
    assert mx <= 2.0 ** -7 * np.max(np.abs(ref))


# ------------------------------------------------------------------ vision tower steps

@CASES
@given(rows=st.integers(1, 300), dim8=st.integers(1, 700), std=scales, shift=st.sampled_from([0.0, 0.5, 20.0]),
       seed=st.integers(0, 2**20))
def test_layer_norm_random_shapes(rows, dim8, std, shift, seed):
    """LayerNorm (weight and bias) on random widths, scales and mean offsets."""
    from oracle import vision as OV
    dim = 8 * dim8
    print(f"layer_norm rows={rows} dim={dim} std={std} shift={shift} seed={seed}", flush=True)
    x = (_randn((rows, dim), seed, std).float() + shift).to(torch.bfloat16)
    w = _gain(dim, seed + 1)
    bb = _randn((dim,), seed + 2, 0.1)
    y = torch.full_like(x, 7.0)
    b.layer_norm(x, w, bb, y, rows, dim)
    torch.cuda.synchronize()
    ref = OV.layer_norm(f64(x), f64(w), f64(bb))
    assert report("layer_norm", f64(y), ref)[0] <= 4e-3


@CASES
@given(shape=gemm_shapes(), act=st.sampled_from([0, 1, 2, "res"]), split=st.booleans(), seed=st.integers(0, 2**20))
def test_linear_bias_random_shapes(shape, act, split, seed):
    """Biased GEMM with GELU (tanh or erf form) or residual on ragged shapes."""
    from oracle import vision as OV
    m, n, k = shape
    print(f"linear_bias m={m} n={n} k={k} act={act} split={split} seed={seed}", flush=True)
    a = _randn((m, k), seed)
    w = _randn((n, k), seed + 1, 0.03)
    bias = _randn((n,), seed + 2, 0.5)
    r = _randn((m, n), seed + 3)
    c = r.clone() if act == "res" else torch.full((m, n), 7.0, device=DEV, dtype=torch.bfloat16)
    ws = torch.empty(b.linear_workspace_bytes(), device=DEV, dtype=torch.uint8) if split else None
    b.linear_bias(a, w, bias, c, m, n, k, act=0 if act == "res" else act,
                  residual=c if act == "res" else None, workspace=ws)
    torch.cuda.synchronize()
    y = OV.linear(f64(a), f64(w), f64(bias))
    ref = {0: y, 1: OV.gelu_tanh(y), 2: OV.gelu_erf(y), "res": y + f64(r)}[act]
    assert report(f"linear_bias act={act}", f64(c), ref)[0] <= 4e-3


@st.composite
def vision_grids(draw):
    """1-4 images / videos of (t, h, w) patches, h and w even (2x2 merge)."""
    n_grids = draw(st.integers(1, 4))
    grids = [(draw(st.integers(1, 3)), 2 * draw(st.integers(1, 10)), 2 * draw(st.integers(1, 10)))
             for _ in range(n_grids)]
    heads = draw(st.integers(1, 4))
    hd = draw(st.sampled_from([64, 72, 80, 96, 128]))
    return grids, heads, hd


@CASES
@given(case=vision_grids(), seed=st.integers(0, 2**20))
def test_vision_attention_random_grids(case, seed):
    """Non-causal attention inside each frame, on random image / video grids,
    head counts and head dims (every (patch, head) row checked)."""
    from oracle import vision as OV
    grids, heads, hd = case
    n = int(sum(t * h * w for t, h, w in grids))
    print(f"vision attention n={n} heads={heads} head_dim={hd} grids={grids} seed={seed}", flush=True)
    q, k, v = (_randn((n, heads, hd), seed + i) for i in range(3))
    sp = b.seq_pad(n)
    q_l = torch.zeros(n, heads, 128, dtype=torch.bfloat16, device=DEV)
    q_l[:, :, :hd] = q
    k_l = torch.zeros(heads, sp, 128, dtype=torch.bfloat16, device=DEV)
    k_l[:, :n, :hd] = k.transpose(0, 1)
    v_pad = torch.zeros(sp, heads, 128, dtype=torch.bfloat16, device=DEV)
    v_pad[:n, :, :hd] = v
    vt_l = v_pad[torch.from_numpy(perm16_tokens(sp)).to(DEV)].permute(1, 2, 0).contiguous()
    o = torch.full((n, heads * hd), 7.0, dtype=torch.bfloat16, device=DEV)
    nb = b.vision_attention_workspace_bytes(n)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    b.vision_attention(q_l, k_l, vt_l, o, n, heads, hd, grids, 2, ws, nb)
    torch.cuda.synchronize()
    ref = OV.segment_attention(f64(q), f64(k), f64(v), OV.segments(grids))
    r, _, w = report_rows("vision attention", f64(o), ref, hd)
    assert r <= 8e-3 and w <= ROW_BAR
