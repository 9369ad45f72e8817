"""Property tests of the CPU oracle over random shapes (hypothesis).

The fixed-case pins check the oracle on hand-picked shapes; these draw the
shapes, scales, positions and rotary sections at random (derandomised: the
same draws every run) and check what must hold for any of them: RMSNorm's
unit output RMS and scale invariance and its agreement with torch's
``rms_norm``; the rotary step's norm preservation and relative-position
property; attention's agreement with torch's causal GQA
``scaled_dot_product_attention``, its row-subset form and its causality; and
the DeepStack add against the dense-buffer form.
"""

import numpy as np
import torch
import torch.nn.functional as F
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

CASES = settings(max_examples=25, deadline=None, derandomize=True, database=None,
                 suppress_health_check=list(HealthCheck))


@CASES
@given(rows=st.integers(1, 9), dim=st.integers(1, 200), log_scale=st.floats(-3, 3), seed=st.integers(0, 2**20))
def test_rmsnorm_unit_rms_and_scale_invariance(rows, dim, log_scale, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(rows, dim)) * 10.0 ** log_scale
    y = oracle.rms_norm(x, np.ones(dim), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-12)
    g = rng.uniform(0.5, 1.5, size=dim)
    np.testing.assert_allclose(oracle.rms_norm(7.5 * x, g, 0.0), oracle.rms_norm(x, g, 0.0), rtol=1e-11, atol=0)


@CASES
@given(rows=st.integers(1, 9), dim=st.integers(1, 200), eps=st.sampled_from([1e-6, 1e-3, 0.5]),
       seed=st.integers(0, 2**20))
def test_rmsnorm_matches_torch(rows, dim, eps, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(rows, dim))
    g = rng.uniform(0.5, 1.5, size=dim)
    ref = F.rms_norm(torch.from_numpy(x), (dim,), torch.from_numpy(g), eps).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, g, eps), ref, rtol=1e-12, atol=1e-14)


@st.composite
def rotary_cases(draw):
    half = draw(st.sampled_from([8, 16, 32, 64]))
    a = draw(st.integers(0, half))
    c = draw(st.integers(0, half - a))
    theta = draw(st.sampled_from([1e4, 1e6, 5e6]))
    return 2 * half, (half - a - c, a, c), theta


@CASES
@given(case=rotary_cases(), seq=st.integers(1, 12), heads=st.integers(1, 4), seed=st.integers(0, 2**20))
def test_rope_preserves_every_rotated_pair(case, seq, heads, seed):
    D, section, theta = case
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(seq, heads, D))
    pos = rng.integers(0, 20000, size=(3, seq))
    cos, sin = oracle.rope_cos_sin(pos, D, theta, section)
    y = oracle.apply_rope(x, cos, sin)
    h = D // 2
    # each (d, d + D/2) pair is rotated, so its length is kept
    np.testing.assert_allclose(np.hypot(y[..., :h], y[..., h:]), np.hypot(x[..., :h], x[..., h:]), rtol=1e-12)


@CASES
@given(case=rotary_cases(), p=st.integers(0, 5000), q_pos=st.integers(0, 5000), shift=st.integers(-3000, 3000),
       seed=st.integers(0, 2**20))
def test_rope_scores_depend_on_position_difference(case, p, q_pos, shift, seed):
    """With all three axes equal (text tokens), <R(p) q, R(p') k> depends on p - p' only."""
    D, section, theta = case
    shift = max(shift, -min(p, q_pos))
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(1, 1, D)); k = rng.normal(size=(1, 1, D))

    def dot(pq, pk):
        cos, sin = oracle.rope_cos_sin(np.array([[pq, pk]] * 3), D, theta, section)
        return float(np.sum(oracle.apply_rope(q, cos[:1], sin[:1]) * oracle.apply_rope(k, cos[1:], sin[1:])))

    assert abs(dot(p, q_pos) - dot(p + shift, q_pos + shift)) <= 1e-9 * (1 + np.linalg.norm(q) * np.linalg.norm(k))


@st.composite
def attention_cases(draw):
    kv = draw(st.integers(1, 3))
    group = draw(st.integers(1, 4))
    S = draw(st.integers(1, 40))
    D = draw(st.sampled_from([4, 16, 32]))
    return S, kv * group, kv, D


@CASES
@given(case=attention_cases(), std=st.sampled_from([0.1, 1.0, 3.0]), seed=st.integers(0, 2**20))
def test_attention_matches_torch_sdpa(case, std, seed):
    S, Hq, Hkv, D = case
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(S, Hq, D)) * std
    k = rng.normal(size=(S, Hkv, D)) * std
    v = rng.normal(size=(S, Hkv, D))
    tq, tk, tv = (torch.from_numpy(a).transpose(0, 1)[None] for a in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)[0].transpose(0, 1)
    got = oracle.causal_gqa_attention(q, k, v, block=int(rng.integers(1, 20)))
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


@CASES
@given(case=attention_cases(), cut=st.integers(0, 39), seed=st.integers(0, 2**20))
def test_attention_rows_and_causality(case, cut, seed):
    S, Hq, Hkv, D = case
    cut = min(cut, S)
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(S, Hq, D)); k = rng.normal(size=(S, Hkv, D)); v = rng.normal(size=(S, Hkv, D))
    full = oracle.causal_gqa_attention(q, k, v)
    rows = np.unique(rng.integers(0, S, size=min(S, 5)))
    np.testing.assert_allclose(oracle.causal_gqa_attention(q, k, v, rows=rows), full[rows], rtol=1e-13, atol=1e-14)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[cut:] += 1.5; k2[cut:] *= -2; v2[cut:] += 4
    assert np.array_equal(oracle.causal_gqa_attention(q2, k2, v2)[:cut], full[:cut])


@CASES
@given(seq=st.integers(1, 60), dim=st.integers(1, 24), density=st.floats(0, 1), seed=st.integers(0, 2**20))
def test_deepstack_equals_dense_buffer_form(seq, dim, density, seed):
    """Adding the features to the masked rows equals adding a zero buffer with
    the features scattered into those rows in order."""
    rng = np.random.default_rng(seed)
    mask = rng.random(seq) < density
    h = rng.normal(size=(seq, dim))
    feat = rng.normal(size=(int(mask.sum()), dim))
    dense = np.zeros((seq, dim))
    dense[np.flatnonzero(mask)] = feat
    np.testing.assert_array_equal(oracle.deepstack_add(h, mask.astype(np.uint8), feat), h + dense)
