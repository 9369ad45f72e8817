"""Per-step parity of the HIP kernels (through the C ABI) against the CPU oracle.

Tolerances follow the arithmetic: every step accumulates in fp32 and rounds
its output to bf16 once (relative rounding error <= 2^-9 per element), so
norms, projections and the rotary step must agree with the float64 oracle to
rel-L2 <= 4e-3; attention additionally rounds the probabilities to bf16 before
the value product, so it gets 8e-3. Inputs are seeded, bf16-valued, and cover
several tiles plus ragged tails.
"""

import numpy as np
import pytest
import torch

import oracle
from multimodal_encoder_prefill_amd import binding as b
from multimodal_encoder_prefill_amd import synth
from helpers import f64, report, report_rows, perm16_tokens

# Largest rel-L2 of any single (token, head) vector: one bf16 rounding of the
# output (and, in attention, of the probabilities) keeps a row near 2^-9;
# a row computed from a wrong head, position or key range is off by O(1).
ROW_BAR = 3e-2

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _randn(shape, seed, std=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * std).to(torch.bfloat16)


def _rand_gain(n, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.rand(n, generator=g, device=DEV) + 0.5).to(torch.bfloat16)


# ------------------------------------------------------------------ RMSNorm

@pytest.mark.parametrize("rows,dim", [(1, 256), (37, 5120), (257, 8192), (4096, 5120)])
def test_rms_norm(rows, dim):
    print(f"rms_norm rows={rows} dim={dim}", flush=True)
    x = _randn((rows, dim), 1, 3.0)
    gamma = _rand_gain(dim, 2)
    y = torch.empty_like(x)
    b.rms_norm(x, gamma, y, rows, dim, 1e-6)
    torch.cuda.synchronize()
    ref = oracle.rms_norm(f64(x), f64(gamma), 1e-6)
    r, _ = report("rms_norm", f64(y), ref)
    assert r <= 4e-3
    assert np.all(np.abs(f64(y) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


def test_rms_norm_in_place():
    x = _randn((64, 5120), 3)
    gamma = _rand_gain(5120, 4)
    ref = oracle.rms_norm(f64(x), f64(gamma), 1e-6)
    b.rms_norm(x, gamma, x, 64, 5120, 1e-6)
    torch.cuda.synchronize()
    assert report("rms_norm in place", f64(x), ref)[0] <= 4e-3


# ------------------------------------------------------------------ GEMMs

GEMM_SHAPES = [
    (64, 64, 64), (300, 96, 128), (256, 256, 256), (513, 1056, 320), (1000, 2048, 1024),
]


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
@pytest.mark.parametrize("residual", [False, True])
def test_linear(m, n, k, residual):
    print(f"linear m={m} n={n} k={k} residual={residual}", flush=True)
    a = _randn((m, k), 10 + m)
    w = _randn((n, k), 20 + n, 0.05)
    c = _randn((m, n), 30) if residual else torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    r0 = f64(c) if residual else 0.0
    b.linear(a, w, c, m, n, k, residual=c if residual else None)
    torch.cuda.synchronize()
    ref = r0 + f64(a) @ f64(w).T
    r, mx = report("linear", f64(c), ref)
    assert r <= 4e-3
    assert mx <= 2.0 ** -7 * np.max(np.abs(ref))


@pytest.mark.parametrize("m,n,k", [(64, 64, 64), (300, 96, 128), (513, 1056, 320)])
def test_linear_swiglu(m, n, k):
    print(f"swiglu m={m} n={n} k={k}", flush=True)
    a = _randn((m, k), 40)
    wg = _randn((n, k), 41, 0.1)
    wu = _randn((n, k), 42, 0.1)
    c = torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    b.linear_swiglu(a, wg, wu, c, m, n, k)
    torch.cuda.synchronize()
    ref = oracle.silu(f64(a) @ f64(wg).T) * (f64(a) @ f64(wu).T)
    r, mx = report("swiglu", f64(c), ref)
    assert r <= 4e-3
    assert mx <= 2.0 ** -7 * np.max(np.abs(ref))


def _gemm_ws():
    return torch.empty(b.linear_workspace_bytes(), device=DEV, dtype=torch.uint8)


@pytest.mark.parametrize("m,n,k,residual", [
    (512, 5120, 8192, True),      # 40 tiles: all split 6 ways along k
    (300, 96, 1024, False),       # ragged m, one partial n tile, 4-way split
    (1000, 2048, 1024, True),     # 32 tiles
    (4096, 5120, 25600, True),    # down projection: 256 tiles of 256 x 320, none split
])
def test_linear_split_k(m, n, k, residual):
    """The last wave of tiles is split along k into fp32 partials and reduced."""
    print(f"linear split-k m={m} n={n} k={k} residual={residual}", flush=True)
    a = _randn((m, k), 12 + m)
    w = _randn((n, k), 13 + n, 0.02)
    c = _randn((m, n), 14) if residual else torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    r0 = f64(c) if residual else 0.0
    c_plain = c.clone()
    b.linear(a, w, c, m, n, k, residual=c if residual else None, workspace=_gemm_ws())
    b.linear(a, w, c_plain, m, n, k, residual=c_plain if residual else None)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, m - 1, 40).astype(int))
    ref = (r0[rows] if residual else 0.0) + f64(a[rows]) @ f64(w).T
    assert report("linear split-k", f64(c)[rows], ref)[0] <= 4e-3
    # split and unsplit differ only by fp32 summation order before one bf16 rounding
    r, mx = report("split vs unsplit", f64(c), f64(c_plain))
    assert r <= 2e-3 and mx <= 2.0 ** -6 * np.max(np.abs(f64(c_plain)))


@pytest.mark.parametrize("m,n,k", [(300, 1056, 1024), (4096, 25600, 5120)])
def test_linear_swiglu_split_k(m, n, k):
    print(f"swiglu split-k m={m} n={n} k={k}", flush=True)
    a = _randn((m, k), 43)
    wg = _randn((n, k), 44, 0.05)
    wu = _randn((n, k), 45, 0.05)
    c = torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    b.linear_swiglu(a, wg, wu, c, m, n, k, workspace=_gemm_ws())
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, m - 1, 24).astype(int))
    ar = f64(a[rows])
    ref = oracle.silu(ar @ f64(wg).T) * (ar @ f64(wu).T)
    assert report("swiglu split-k", f64(c)[rows], ref)[0] <= 4e-3


@pytest.mark.parametrize("name,m,n,k", [("o_proj", 4096, 5120, 8192), ("down", 4096, 5120, 25600),
                                         ("qkv", 4096, 10240, 5120)])
def test_linear_full_size_sampled_rows(name, m, n, k):
    """Full-size shapes as the prefill runs them; the oracle checks sampled rows."""
    print(f"linear full {name} m={m} n={n} k={k}", flush=True)
    a = _randn((m, k), 50)
    w = _randn((n, k), 51, 0.02)
    c = _randn((m, n), 52)
    r0 = f64(c)
    b.linear(a, w, c, m, n, k, residual=c)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 1000, 2047, 3333, m - 1])
    ref = r0[rows] + f64(a[rows]) @ f64(w).T
    assert report(f"{name} sampled", f64(c)[rows], ref)[0] <= 4e-3


@pytest.mark.parametrize("m,n,k,residual", [
    (4000, 5120, 320, True),     # 16 x 16 tiles of 256 x 320, ragged last m-tile
    (4096, 10240, 192, False),   # 16 x 32 tiles
])
def test_linear_wide_tiles_dense(m, n, k, residual):
    """Shapes whose 320-wide tiles fill whole waves of the chip, every output
    against the oracle."""
    print(f"linear wide m={m} n={n} k={k} residual={residual}", flush=True)
    a = _randn((m, k), 70)
    w = _randn((n, k), 71, 0.05)
    c = _randn((m, n), 72) if residual else torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    r0 = f64(c) if residual else 0.0
    b.linear(a, w, c, m, n, k, residual=c if residual else None, workspace=_gemm_ws())
    torch.cuda.synchronize()
    ref = r0 + f64(a) @ f64(w).T
    r, mx = report("linear wide", f64(c), ref)
    assert r <= 4e-3
    assert mx <= 2.0 ** -7 * np.max(np.abs(ref))


def test_swiglu_wide_tiles_dense():
    """gate/up with 320-row tiles (gate and up rows interleaved in 8-row
    groups inside each 32-row block), every output against the oracle."""
    m, n, k = 4000, 25600, 192
    a = _randn((m, k), 73)
    wg = _randn((n, k), 74, 0.1)
    wu = _randn((n, k), 75, 0.1)
    c = torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    b.linear_swiglu(a, wg, wu, c, m, n, k, workspace=_gemm_ws())
    torch.cuda.synchronize()
    ar = f64(a)
    ref = oracle.silu(ar @ f64(wg).T) * (ar @ f64(wu).T)
    r, mx = report("swiglu wide", f64(c), ref)
    assert r <= 4e-3
    assert mx <= 2.0 ** -7 * np.max(np.abs(ref))


def test_swiglu_full_size_sampled_rows():
    m, n, k = 4096, 25600, 5120
    a = _randn((m, k), 60)
    wg = _randn((n, k), 61, 0.02)
    wu = _randn((n, k), 62, 0.02)
    c = torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    b.linear_swiglu(a, wg, wu, c, m, n, k)
    torch.cuda.synchronize()
    rows = np.array([0, 17, 511, 2048, 4095])
    ar = f64(a[rows])
    ref = oracle.silu(ar @ f64(wg).T) * (ar @ f64(wu).T)
    assert report("swiglu full sampled", f64(c)[rows], ref)[0] <= 4e-3


# ------------------------------------------------------------------ q/k norm + rotary

def _qk_case(dims, seq, positions, seed):
    qw, kvw = dims.q_width, dims.kv_width
    qkv = _randn((seq, qw + 2 * kvw), seed, 2.0)
    qn = _rand_gain(dims.head_dim, seed + 1)
    kn = _rand_gain(dims.head_dim, seed + 2)
    sp = b.seq_pad(seq)
    q_out = torch.full((seq, dims.n_heads, dims.head_dim), 7.0, device=DEV, dtype=torch.bfloat16)
    k_out = torch.full((dims.n_kv_heads, sp, dims.head_dim), 7.0, device=DEV, dtype=torch.bfloat16)
    vt_out = torch.full((dims.n_kv_heads, dims.head_dim, sp), 7.0, device=DEV, dtype=torch.bfloat16)
    pos = torch.from_numpy(np.ascontiguousarray(positions, dtype=np.int32)).to(DEV)
    cfg = b.config_from_dims(dims)
    b.qk_norm_rope(cfg, qkv, qn, kn, pos, seq, q_out, k_out, vt_out)
    torch.cuda.synchronize()
    x = f64(qkv)
    D = dims.head_dim
    cos, sin = oracle.rope_cos_sin(positions, D, dims.rope_theta, dims.mrope_section)
    q_ref = oracle.apply_rope(oracle.rms_norm(x[:, :qw].reshape(seq, -1, D), f64(qn), dims.rms_eps), cos, sin)
    k_ref = oracle.apply_rope(oracle.rms_norm(x[:, qw:qw + kvw].reshape(seq, -1, D), f64(kn), dims.rms_eps), cos, sin)
    v_ref = x[:, qw + kvw:].reshape(seq, -1, D)
    _qk_case.inputs = dict(qkv=qkv, qn=qn, pos=pos, cfg=cfg)
    return q_out, k_out, vt_out, q_ref, k_ref, v_ref, sp


@pytest.mark.parametrize("key,seq", [("tiny", 64), ("tiny", 77), ("full", 100), ("full", 2048)])
def test_qk_norm_rope(key, seq):
    print(f"qk_norm_rope {key} seq={seq}", flush=True)
    dims = synth.TINY if key == "tiny" else synth.FULL
    positions = synth.random_positions(seq, 3000, seed=seq)
    q_out, k_out, vt_out, q_ref, k_ref, v_ref, sp = _qk_case(dims, seq, positions, 70 + seq)
    D = dims.head_dim
    r, _, w = report_rows("q", f64(q_out), q_ref, D)
    assert r <= 4e-3 and w <= ROW_BAR
    kk = f64(k_out)
    r, _, w = report_rows("k", kk[:, :seq].transpose(1, 0, 2), k_ref, D)
    assert r <= 4e-3 and w <= ROW_BAR
    assert np.all(kk[:, seq:] == 0)
    vt = f64(vt_out)                          # [Hkv, D, sp], permuted columns
    tok = perm16_tokens(sp)
    v_pad = np.zeros((sp,) + v_ref.shape[1:])
    v_pad[:seq] = v_ref
    assert np.array_equal(vt, v_pad[tok].transpose(1, 2, 0))   # a pure relayout: exact


def test_qk_norm_rope_workload_positions():
    """Image-layout positions of the 4096-token workload (text / 1x32x64 grid / text)."""
    wl = synth.WORKLOADS["image_s4096_l50"]
    q_out, k_out, _, q_ref, k_ref, _, _ = _qk_case(wl.dims, wl.seq, synth.positions(wl), 90)
    D = wl.dims.head_dim
    r, _, w = report_rows("q image", f64(q_out), q_ref, D)
    assert r <= 4e-3 and w <= ROW_BAR
    r, _, w = report_rows("k image", f64(k_out)[:, :wl.seq].transpose(1, 0, 2), k_ref, D)
    assert r <= 4e-3 and w <= ROW_BAR


# ------------------------------------------------------------------ attention

def _attn_inputs(seq, hq, hkv, d, seed):
    q = _randn((seq, hq, d), seed)
    k = _randn((seq, hkv, d), seed + 1)
    v = _randn((seq, hkv, d), seed + 2)
    sp = b.seq_pad(seq)
    k_l = torch.zeros((hkv, sp, d), device=DEV, dtype=torch.bfloat16)
    k_l[:, :seq] = k.transpose(0, 1)
    v_pad = torch.zeros((sp, hkv, d), device=DEV, dtype=torch.bfloat16)
    v_pad[:seq] = v
    tok = torch.from_numpy(perm16_tokens(sp)).to(DEV)
    vt_l = v_pad[tok].permute(1, 2, 0).contiguous()
    return q, k, v, k_l, vt_l


@pytest.mark.parametrize("seq,hq,hkv,d", [
    (1, 4, 1, 64), (31, 4, 1, 64), (64, 4, 1, 64), (100, 8, 1, 128), (257, 16, 2, 128),
    (200, 8, 4, 128), (130, 2, 2, 64), (700, 64, 8, 128),
])
def test_attention(seq, hq, hkv, d):
    print(f"attention seq={seq} heads={hq}/{hkv} d={d}", flush=True)
    q, k, v, k_l, vt_l = _attn_inputs(seq, hq, hkv, d, 100 + seq)
    o = torch.empty((seq, hq * d), device=DEV, dtype=torch.bfloat16)
    b.attention(q, k_l, vt_l, o, seq, hq, hkv, d)
    torch.cuda.synchronize()
    ref = oracle.causal_gqa_attention(f64(q), f64(k), f64(v)).reshape(seq, hq * d)
    r, _, w = report_rows("attention", f64(o), ref, d)
    assert r <= 8e-3 and w <= ROW_BAR


@pytest.mark.parametrize("seq", [1, 32, 33, 64, 65, 96, 127, 128, 129, 191, 256])
def test_attention_group8_tile_edges(seq):
    """8 query heads per key/value head at head_dim 128 around the 32-query
    block and key-tile boundaries: one to three key tiles, the masked last
    tile at both offsets of a query block, ragged ends."""
    print(f"attention g8 seq={seq}", flush=True)
    hq, hkv, d = 16, 2, 128
    q, k, v, k_l, vt_l = _attn_inputs(seq, hq, hkv, d, 300 + seq)
    o = torch.empty((seq, hq * d), device=DEV, dtype=torch.bfloat16)
    b.attention(q, k_l, vt_l, o, seq, hq, hkv, d)
    torch.cuda.synchronize()
    ref = oracle.causal_gqa_attention(f64(q), f64(k), f64(v)).reshape(seq, hq * d)
    r, _, w = report_rows("attention g8", f64(o), ref, d)
    assert r <= 8e-3 and w <= ROW_BAR


def test_attention_rising_scores_rescale():
    """Keys whose scale grows along the sequence, so the running maximum of
    most queries rises by far more than the lazy threshold on later tiles and
    the earlier output is rescaled many times."""
    seq, hq, hkv, d = 600, 8, 1, 128
    q, k, v, k_l, vt_l = _attn_inputs(seq, hq, hkv, d, 17)
    ramp = torch.linspace(0.05, 20.0, seq, device=DEV).reshape(seq, 1, 1)
    k = (k.float() * ramp).to(torch.bfloat16)
    k_l[:, :seq] = k.transpose(0, 1)
    o = torch.empty((seq, hq * d), device=DEV, dtype=torch.bfloat16)
    b.attention(q, k_l, vt_l, o, seq, hq, hkv, d)
    torch.cuda.synchronize()
    ref = oracle.causal_gqa_attention(f64(q), f64(k), f64(v)).reshape(seq, hq * d)
    r, _, w = report_rows("attention rising", f64(o), ref, d)
    assert r <= 8e-3 and w <= ROW_BAR


def test_attention_full_size_sampled_rows():
    seq, hq, hkv, d = 4096, 64, 8, 128
    q, k, v, k_l, vt_l = _attn_inputs(seq, hq, hkv, d, 7)
    o = torch.empty((seq, hq * d), device=DEV, dtype=torch.bfloat16)
    b.attention(q, k_l, vt_l, o, seq, hq, hkv, d)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 1000, 2047, 2048, 4095])
    ref = oracle.causal_gqa_attention(f64(q), f64(k), f64(v), rows=rows).reshape(len(rows), -1)
    r, _, w = report_rows("attention full sampled", f64(o)[rows], ref, d)
    assert r <= 8e-3 and w <= ROW_BAR


def test_attention_causal_bitwise():
    """Changing tokens after position c leaves earlier outputs bit-identical."""
    seq, hq, hkv, d, cut = 300, 8, 1, 128, 150
    q, k, v, k_l, vt_l = _attn_inputs(seq, hq, hkv, d, 11)
    o1 = torch.empty((seq, hq * d), device=DEV, dtype=torch.bfloat16)
    b.attention(q, k_l, vt_l, o1, seq, hq, hkv, d)
    q2 = q.clone(); q2[cut:] *= 2
    k_l2 = k_l.clone(); k_l2[:, cut:] = -k_l2[:, cut:]
    vt2 = vt_l.clone()
    cols = torch.from_numpy(np.flatnonzero(perm16_tokens(b.seq_pad(seq)) >= cut)).to(DEV)
    vt2[:, :, cols] += 1.0
    o2 = torch.empty_like(o1)
    b.attention(q2, k_l2, vt2, o2, seq, hq, hkv, d)
    torch.cuda.synchronize()
    assert torch.equal(o1[:cut], o2[:cut])
    assert not torch.equal(o1[cut:], o2[cut:])


# ------------------------------------------------------------------ attention, q norm + rotary fused

def _qnorm_attention_case(dims, seq, positions, seed, rows=None):
    """The decoder layer's form of the attention step (q read raw from the
    q/k/v projection output, normalised and rotated in the attention kernel)
    next to the two-step chain, and the oracle's q/k norm, rotary and causal
    GQA attention on the same q/k/v rows."""
    q_out, k_out, vt_out, q_ref, k_ref, v_ref, _ = _qk_case(dims, seq, positions, seed)
    inp = _qk_case.inputs
    D, hq, hkv = dims.head_dim, dims.n_heads, dims.n_kv_heads
    nbytes = b.qnorm_attention_workspace_bytes(inp["cfg"], seq)
    ws = torch.empty(nbytes, device=DEV, dtype=torch.uint8)
    o = torch.full((seq, hq * D), 7.0, device=DEV, dtype=torch.bfloat16)
    b.qnorm_attention(inp["cfg"], inp["qkv"], inp["qn"], inp["pos"], k_out, vt_out, o, seq, ws, nbytes)
    o_chain = torch.empty_like(o)
    b.attention(q_out, k_out, vt_out, o_chain, seq, hq, hkv, D)
    torch.cuda.synchronize()
    r = np.arange(seq) if rows is None else rows
    ref = oracle.causal_gqa_attention(q_ref, k_ref, v_ref, rows=rows).reshape(len(r), hq * D)
    return f64(o)[r], f64(o_chain)[r], ref


@pytest.mark.parametrize("key,seq", [("tiny", 64), ("tiny", 77), ("full", 100), ("full", 700)])
def test_qnorm_attention(key, seq):
    print(f"qnorm_attention {key} seq={seq}", flush=True)
    dims = synth.TINY if key == "tiny" else synth.FULL
    positions = synth.random_positions(seq, 3000, seed=seq + 5)
    got, chain, ref = _qnorm_attention_case(dims, seq, positions, 500 + seq)
    r, _, w = report_rows("qnorm attention", got, ref, dims.head_dim)
    assert r <= 8e-3 and w <= ROW_BAR
    # the two-step chain rounds the same q once too; only the order of the
    # q row's sum of squares differs
    assert report("qnorm attention vs chain", got, chain)[0] <= 4e-3


def test_qnorm_attention_workload_sampled_rows():
    """4096 tokens, 64/8 heads of 128, the image workload's positions, rows
    sampled over the sequence and at the image block's edges."""
    wl = synth.WORKLOADS["image_s4096_l50"]
    vis = np.flatnonzero(synth.visual_mask(wl))
    rows = np.unique(np.array([0, 1, 63, 64, vis[0] - 1, vis[0], vis[0] + 64, vis[-1], vis[-1] + 1,
                               3000, wl.seq - 1]))
    got, chain, ref = _qnorm_attention_case(wl.dims, wl.seq, synth.positions(wl), 95, rows)
    r, _, w = report_rows("qnorm attention image sampled", got, ref, wl.dims.head_dim)
    assert r <= 8e-3 and w <= ROW_BAR
    assert report("qnorm attention image vs chain", got, chain)[0] <= 4e-3


# ------------------------------------------------------------------ DeepStack

@pytest.mark.parametrize("seq,dim,density", [(64, 256, 0.5), (4096, 5120, 0.5), (333, 5120, 0.1)])
def test_deepstack_inject(seq, dim, density):
    print(f"deepstack seq={seq} dim={dim}", flush=True)
    rng = np.random.default_rng(seq)
    mask = (rng.random(seq) < density).astype(np.uint8)
    n_vis = int(mask.sum())
    h = _randn((seq, dim), 200)
    feat = _randn((max(n_vis, 1), dim), 201)
    ref = oracle.deepstack_add(f64(h), mask, f64(feat)[:n_vis])
    ws = torch.empty(seq * 4 + 512, device=DEV, dtype=torch.uint8)
    m = torch.from_numpy(mask).to(DEV)
    b.deepstack_inject(h, seq, dim, m, n_vis, feat, ws, ws.numel())
    torch.cuda.synchronize()
    got = f64(h)
    assert report("deepstack", got, ref)[0] <= 4e-3
    untouched = mask == 0
    assert np.array_equal(got[untouched], ref[untouched])   # non-visual rows unchanged
    assert b.count_visual(m, seq, ws, ws.numel()) == n_vis


def test_deepstack_short_and_long_masks_stay_in_bounds():
    seq, dim = 128, 256
    mask = np.zeros(seq, np.uint8); mask[10:20] = 1        # 10 visual tokens
    h0 = _randn((seq, dim), 300)
    feat = _randn((16, dim), 301)
    ws = torch.empty(seq * 4 + 512, device=DEV, dtype=torch.uint8)
    m = torch.from_numpy(mask).to(DEV)
    h = h0.clone()
    b.deepstack_inject(h, seq, dim, m, 16, feat, ws, ws.numel())      # n_vis > popcount
    h2 = h0.clone()
    b.deepstack_inject(h2, seq, dim, m, 4, feat, ws, ws.numel())      # n_vis < popcount
    torch.cuda.synchronize()
    ref16 = f64(h0); ref16[10:20] += f64(feat)[:10]
    ref4 = f64(h0); ref4[10:14] += f64(feat)[:4]
    assert report("long mask", f64(h), ref16)[0] <= 4e-3
    assert report("short mask", f64(h2), ref4)[0] <= 4e-3
    assert np.array_equal(f64(h2)[14:], f64(h0)[14:])
