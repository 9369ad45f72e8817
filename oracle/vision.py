"""Qwen3-VL vision tower, as plain float64 reference code.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

H3 encoder page, ``MiniMaxH3Qwen3VLVisionModel`` and its parts:

* patch embedding: a Conv3d whose kernel equals its stride, i.e. every patch
  (in_channels x temporal_patch x patch x patch values, flattened in that
  order) times the flattened kernel, plus the bias
  (``MiniMaxH3Qwen3VLVisionPatchEmbed``);
* learned position embeddings bilinearly interpolated from a square table
  to each image's patch grid and reordered so every merge x merge block of
  patches is consecutive (``fast_pos_embed_interpolate``);
* 2-D rotary position: row and column of each patch (same block order) times
  the inverse frequencies of a head_dim/2 rotary with theta 10000; the row
  and column angles are concatenated, then duplicated to head_dim, and the
  usual rotate-half is applied to q and k in fp32 (``rot_pos_emb``,
  ``MiniMaxH3Qwen3VLVisionRotaryEmbedding``, ``_apply_rotary_pos_emb_vision``);
* blocks: x + attn(LayerNorm(x)), then x + MLP(LayerNorm(x)); attention is
  multi-head, non-causal, within each frame of each image only (cu_seqlens),
  scale 1/sqrt(head_dim); the MLP is fc2(gelu_tanh(fc1(x))), all linears with
  bias (``MiniMaxH3Qwen3VLVisionBlock`` and its attention / MLP);
* after the blocks listed in deepstack_visual_indexes a DeepStack merger, and
  after the last block the main merger: groups of merge^2 consecutive tokens
  are concatenated; the main merger normalises before concatenation, the
  DeepStack mergers after; then fc2(gelu_erf(fc1(x))) with biases
  (``MiniMaxH3Qwen3VLVisionPatchMerger``).

LayerNorm eps is 1e-6 everywhere on the page.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Sequence, Tuple

import numpy as np
from scipy.special import erf

LN_EPS = 1e-6
ROPE_THETA = 10000.0


@dataclass(frozen=True)
class VisionDims:
    hidden: int
    n_heads: int
    intermediate: int
    depth: int
    patch: int
    temporal_patch: int
    in_channels: int
    merge: int
    out_hidden: int
    pos_side: int            # sqrt(num_position_embeddings)
    deepstack: Tuple[int, ...]

    @property
    def head_dim(self) -> int:
        return self.hidden // self.n_heads

    @property
    def patch_dim(self) -> int:
        return self.in_channels * self.temporal_patch * self.patch * self.patch

    @property
    def merged_hidden(self) -> int:
        return self.hidden * self.merge * self.merge


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def layer_norm(x, w, b, eps: float = LN_EPS) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) * w + b over the last axis (biased variance)."""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * _f64(w) + _f64(b)


def gelu_tanh(x) -> np.ndarray:
    x = _f64(x)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def gelu_erf(x) -> np.ndarray:
    x = _f64(x)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def linear(x, w, b=None) -> np.ndarray:
    y = _f64(x) @ _f64(w).T
    return y if b is None else y + _f64(b)


def patch_embed(pixels, w, b) -> np.ndarray:
    """pixels [n, C*T*P*P] (C, T, P, P order), w [hidden, C, T, P, P], b [hidden]."""
    w = _f64(w)
    return linear(pixels, w.reshape(w.shape[0], -1), b)


def _block_order(t: int, h: int, w: int, m: int) -> List[Tuple[int, int, int]]:
    """(frame, row, col) of each patch in the order the tower keeps them: frames,
    then merge x merge blocks row-major, then rows and columns inside a block."""
    out = []
    for f in range(t):
        for br in range(h // m):
            for bc in range(w // m):
                for ir in range(m):
                    for ic in range(m):
                        out.append((f, br * m + ir, bc * m + ic))
    return out


def pos_embed_interpolate(table, grids: Sequence[Sequence[int]], pos_side: int,
                          merge: int) -> np.ndarray:
    """[sum t*h*w, hidden] interpolated position embeddings, in block order.

    Patch row r of an h-row grid samples the table at the fractional row
    r*(pos_side-1)/(h-1) (torch.linspace); the four neighbours floor / floor+1
    (clipped to the table) are mixed bilinearly; columns likewise."""
    table = _f64(table)
    rows = []
    for t, h, w in grids:
        hs = np.linspace(0.0, pos_side - 1, h, dtype=np.float32).astype(np.float64)
        ws = np.linspace(0.0, pos_side - 1, w, dtype=np.float32).astype(np.float64)
        for (f, r, c) in _block_order(t, h, w, merge):
            y, x = hs[r], ws[c]
            y0, x0 = int(y), int(x)
            y1, x1 = min(y0 + 1, pos_side - 1), min(x0 + 1, pos_side - 1)
            dy, dx = y - y0, x - x0
            rows.append((1 - dy) * (1 - dx) * table[y0 * pos_side + x0]
                        + (1 - dy) * dx * table[y0 * pos_side + x1]
                        + dy * (1 - dx) * table[y1 * pos_side + x0]
                        + dy * dx * table[y1 * pos_side + x1])
    return np.asarray(rows)


def rotary_angles(grids: Sequence[Sequence[int]], head_dim: int, merge: int) -> np.ndarray:
    """[n, head_dim] angles: [row*f, col*f] with f_j = theta^(-2j/(head_dim/2)),
    j < head_dim/4, then the same head_dim/2 angles again."""
    half = head_dim // 2
    inv = 1.0 / (ROPE_THETA ** (np.arange(0, half, 2, dtype=np.float64) / half))
    out = []
    for t, h, w in grids:
        for (_, r, c) in _block_order(t, h, w, merge):
            a = np.concatenate([r * inv, c * inv])
            out.append(np.concatenate([a, a]))
    return np.asarray(out)


def rope(x, ang) -> np.ndarray:
    """Rotate-half rotary over the last axis of x [n, heads, D] with angles [n, D]."""
    x = _f64(x)
    d2 = x.shape[-1] // 2
    rot = np.concatenate([-x[..., d2:], x[..., :d2]], axis=-1)
    return x * np.cos(ang)[:, None, :] + rot * np.sin(ang)[:, None, :]


def segments(grids: Sequence[Sequence[int]]) -> List[Tuple[int, int]]:
    """[start, end) token ranges of the frames (cu_seqlens)."""
    out, s = [], 0
    for t, h, w in grids:
        for _ in range(t):
            out.append((s, s + h * w))
            s += h * w
    return out


def segment_attention(q, k, v, segs) -> np.ndarray:
    """q, k, v [n, heads, D] -> [n, heads*D]; softmax(q k^T / sqrt(D)) v within each segment."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, H, D = q.shape
    out = np.zeros((n, H, D))
    for (s, e) in segs:
        for h in range(H):
            sc = q[s:e, h] @ k[s:e, h].T / math.sqrt(D)
            sc -= sc.max(axis=1, keepdims=True)
            p = np.exp(sc)
            p /= p.sum(axis=1, keepdims=True)
            out[s:e, h] = p @ v[s:e, h]
    return out.reshape(n, H * D)


def block(x, p: Dict[str, np.ndarray], dims: VisionDims, ang, segs) -> np.ndarray:
    """One vision block; p holds norm1_w/b, qkv_w/b, proj_w/b, norm2_w/b, fc1_w/b, fc2_w/b."""
    x = _f64(x)
    n, H, D = x.shape[0], dims.n_heads, dims.head_dim
    u = layer_norm(x, p["norm1_w"], p["norm1_b"])
    qkv = linear(u, p["qkv_w"], p["qkv_b"]).reshape(n, 3, H, D)
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    q, k = rope(q, ang), rope(k, ang)
    x = x + linear(segment_attention(q, k, v, segs), p["proj_w"], p["proj_b"])
    u = layer_norm(x, p["norm2_w"], p["norm2_b"])
    return x + linear(gelu_tanh(linear(u, p["fc1_w"], p["fc1_b"])), p["fc2_w"], p["fc2_b"])


def merger(x, p: Dict[str, np.ndarray], dims: VisionDims, postshuffle: bool) -> np.ndarray:
    """p holds norm_w/b, fc1_w/b, fc2_w/b; x [n, hidden] -> [n / merge^2, out_hidden]."""
    x = _f64(x)
    mh = dims.merged_hidden
    if postshuffle:
        u = layer_norm(x.reshape(-1, mh), p["norm_w"], p["norm_b"])
    else:
        u = layer_norm(x, p["norm_w"], p["norm_b"]).reshape(-1, mh)
    return linear(gelu_erf(linear(u, p["fc1_w"], p["fc1_b"])), p["fc2_w"], p["fc2_b"])


def forward(pixels, grids: Sequence[Sequence[int]], weights: Dict, dims: VisionDims,
            return_blocks: bool = False):
    """(merged [n/merge^2, out_hidden], DeepStack list) for patches of `grids`.

    weights: "patch_w", "patch_b", "pos_table", "blocks" (list of block dicts),
    "merger" (dict), "deepstack" (list of merger dicts)."""
    x = patch_embed(pixels, weights["patch_w"], weights["patch_b"])
    x = x + pos_embed_interpolate(weights["pos_table"], grids, dims.pos_side, dims.merge)
    ang = rotary_angles(grids, dims.head_dim, dims.merge)
    segs = segments(grids)
    ds, states = [], [x]
    for i, p in enumerate(weights["blocks"]):
        x = block(x, p, dims, ang, segs)
        states.append(x)
        if i in dims.deepstack:
            ds.append(merger(x, weights["deepstack"][dims.deepstack.index(i)], dims, True))
    out = merger(x, weights["merger"], dims, False)
    return (out, ds, states) if return_blocks else (out, ds)
