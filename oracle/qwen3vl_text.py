"""Float64 reference of the Qwen3-VL text decoder as the MiniMax H3 encoder runs it.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

What is computed (H3 encoder page, ``MiniMaxH3Qwen3VLTextModel.forward`` and
the module docstring's computation contract): starting from the input
embeddings, run the first ``n_layers`` decoder layers; after decoder layer
``l`` for ``l`` below the number of DeepStack levels, add level ``l``'s visual
features to the visual-token rows; return the hidden state after the last
layer with no final norm.

Everything is float64. Matrix products use ``numpy.matmul`` as a library
primitive; nothing is blocked, fused or reordered beyond the plain definition,
except that attention walks the query rows in blocks (exact softmax per row,
so the result is the same up to rounding order).

Notation: S tokens, H hidden, Hq query heads, Hkv key/value heads, D head dim,
I MLP intermediate width. Weights follow the ``F.linear`` convention
``y = x @ W.T`` with ``W`` stored ``[out, in]``.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np


@dataclass(frozen=True)
class ModelDims:
    """Shape constants of the text decoder.

    H3 encoder page: ``MINIMAX_H3_QWEN3VL_HIDDEN_DIM`` (5120) and
    ``MINIMAX_H3_QWEN3VL_SELECTED_LM_LAYER`` (50); the head counts, head dim,
    intermediate width, eps and rope theta come from the Qwen3-VL config
    object that the page reads (``config.num_attention_heads`` etc.).
    """

    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    rms_eps: float = 1e-6
    rope_theta: float = 5e6
    mrope_section: tuple = (24, 20, 20)


@dataclass
class LayerWeights:
    """One decoder layer's parameters as float64 arrays.

    H3 encoder page, ``MiniMaxH3Qwen3VLTextDecoderLayer`` /
    ``MiniMaxH3Qwen3VLTextAttention`` / ``MiniMaxH3Qwen3VLTextMLP``:
    q/k/v are the three row slices of the fused qkv weight, gate/up the two
    row slices of the fused gate_up weight.
    """

    ln_in: np.ndarray    # [H]      input_layernorm gamma
    w_q: np.ndarray      # [Hq*D, H]
    w_k: np.ndarray      # [Hkv*D, H]
    w_v: np.ndarray      # [Hkv*D, H]
    q_norm: np.ndarray   # [D]
    k_norm: np.ndarray   # [D]
    w_o: np.ndarray      # [H, Hq*D]
    ln_post: np.ndarray  # [H]      post_attention_layernorm gamma
    w_gate: np.ndarray   # [I, H]
    w_up: np.ndarray     # [I, H]
    w_down: np.ndarray   # [H, I]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """Root-mean-square normalisation over the last axis, then a per-channel gain.

    H3 encoder page, ``MiniMaxH3Qwen3VLRMSNorm``: the variance (mean of
    squares, no mean subtraction) and the scaling are taken in full
    precision, and the result is multiplied by the learned gamma.
    """
    x = _f64(x)
    mean_square = np.mean(np.square(x), axis=-1, keepdims=True)
    return _f64(gamma) * (x / np.sqrt(mean_square + eps))


def mrope_slot_axes(half_dim: int, section: Sequence[int]) -> np.ndarray:
    """Which position axis (0=T, 1=H, 2=W) drives each rotary frequency slot.

    H3 encoder page, ``_apply_interleaved_mrope``: the chunked T/H/W
    frequency layout is turned into an interleaved one. Slot ``j`` uses the
    H axis when ``j % 3 == 1`` and ``j < 3 * section[1]``, the W axis when
    ``j % 3 == 2`` and ``j < 3 * section[2]``, and the T axis otherwise.
    """
    axes = np.zeros(half_dim, dtype=np.int64)
    for j in range(half_dim):
        if j % 3 == 1 and j < 3 * section[1]:
            axes[j] = 1
        elif j % 3 == 2 and j < 3 * section[2]:
            axes[j] = 2
    return axes


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Inverse frequencies theta^(-2j/D), j < D/2.

    H3 encoder page, ``MiniMaxH3Qwen3VLTextRotaryEmbedding._get_inv_freq``.
    """
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / head_dim)


def rope_cos_sin(positions, head_dim: int, theta: float, section: Sequence[int]):
    """Cosine/sine tables [S, D] for 3-axis positions [3, S].

    H3 encoder page, ``MiniMaxH3Qwen3VLTextRotaryEmbedding.forward``: the
    angle of slot j at token s is ``pos[axis(j), s] * inv_freq[j]``; the slot
    angles are duplicated (first half and second half of the head use the same
    angles) before taking cos and sin.
    """
    pos = np.asarray(positions, dtype=np.float64)
    if pos.ndim != 2 or pos.shape[0] != 3:
        raise ValueError(f"positions must be [3, S], got {pos.shape}")
    half = head_dim // 2
    axes = mrope_slot_axes(half, section)
    inv_freq = rope_inv_freq(head_dim, theta)
    angle = pos[axes, :].T * inv_freq[None, :]          # [S, half]
    angle = np.concatenate([angle, angle], axis=-1)      # [S, D]
    return np.cos(angle), np.sin(angle)


def apply_rope(x, cos, sin) -> np.ndarray:
    """Rotate-half rotary embedding of x [S, heads, D] with tables [S, D].

    H3 encoder page, ``_rotate_half`` and ``_apply_rotary_pos_emb``: the
    rotated-half of x is (-second half, first half); the output is
    ``x * cos + rotated_half(x) * sin``, tables broadcast over heads.
    """
    x = _f64(x)
    half = x.shape[-1] // 2
    rotated = np.concatenate([-x[..., half:], x[..., :half]], axis=-1)
    return x * cos[:, None, :] + rotated * sin[:, None, :]


def silu(z) -> np.ndarray:
    """SiLU z * sigmoid(z) (``F.silu`` in ``MiniMaxH3Qwen3VLTextMLP.forward``)."""
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def causal_gqa_attention(q, k, v, rows: Optional[np.ndarray] = None, block: int = 512) -> np.ndarray:
    """Causal grouped-query attention with the default 1/sqrt(D) scale.

    H3 encoder page, ``MiniMaxH3Qwen3VLTextAttention.forward``: K and V are
    expanded to the query-head count with ``repeat_interleave`` (query head h
    reads key/value head ``h // (Hq // Hkv)``), then scaled dot-product
    attention with ``is_causal=True`` (key j is visible to query i iff
    j <= i) and no explicit scale, i.e. 1/sqrt(D). The padding mask is all
    ones (module docstring), so causality is the only mask.

    q [S, Hq, D], k and v [S, Hkv, D]. ``rows`` (sorted, unique) restricts the
    output to those query rows; the result is then [len(rows), Hq, D].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    group = Hq // Hkv
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), Hq, D), dtype=np.float64)
    scale = 1.0 / np.sqrt(D)
    for start in range(0, len(rows), block):
        r = rows[start:start + block]
        n_keys = int(r[-1]) + 1
        visible = np.arange(n_keys)[None, :] <= r[:, None]          # [b, n_keys]
        for h in range(Hq):
            g = h // group
            logits = (q[r, h, :] @ k[:n_keys, g, :].T) * scale
            logits = np.where(visible, logits, -np.inf)
            logits = logits - logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p = p / p.sum(axis=1, keepdims=True)
            out[start:start + len(r), h, :] = p @ v[:n_keys, g, :]
    return out


def decoder_layer(h, w: LayerWeights, cos, sin, dims: ModelDims,
                  rows: Optional[np.ndarray] = None) -> np.ndarray:
    """One decoder layer on hidden state h [S, H].

    H3 encoder page, ``MiniMaxH3Qwen3VLTextDecoderLayer.forward`` with
    ``MiniMaxH3Qwen3VLTextAttention.forward`` and
    ``MiniMaxH3Qwen3VLTextMLP.forward``:

    1. u = rms(h, input_layernorm)
    2. q, k, v = u W_q^T, u W_k^T, u W_v^T, viewed as heads of D
    3. per-head rms over D with q_norm / k_norm, then rotary on q and k
    4. causal GQA attention, heads concatenated (column h*D + d)
    5. h1 = h + attn @ W_o^T
    6. u2 = rms(h1, post_attention_layernorm)
    7. out = h1 + (silu(u2 W_gate^T) * (u2 W_up^T)) @ W_down^T

    ``rows`` restricts the output to those rows (K and V still cover every
    token up to the last requested row); the result is then [len(rows), H].
    """
    h = _f64(h)
    S = h.shape[0]
    D, Hq, Hkv = dims.head_dim, dims.n_heads, dims.n_kv_heads
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    n_ctx = int(rows[-1]) + 1 if len(rows) else 0

    u = rms_norm(h[:n_ctx], w.ln_in, dims.rms_eps)
    k = (u @ _f64(w.w_k).T).reshape(n_ctx, Hkv, D)
    v = (u @ _f64(w.w_v).T).reshape(n_ctx, Hkv, D)
    q = (u[rows] @ _f64(w.w_q).T).reshape(len(rows), Hq, D)

    q = rms_norm(q, w.q_norm, dims.rms_eps)
    k = rms_norm(k, w.k_norm, dims.rms_eps)
    q = apply_rope(q, cos[rows], sin[rows])
    k = apply_rope(k, cos[:n_ctx], sin[:n_ctx])

    # Scatter the requested queries into a full-length array so attention can
    # index them by token position.
    q_full = np.zeros((n_ctx, Hq, D), dtype=np.float64)
    q_full[rows] = q
    attn = causal_gqa_attention(q_full, k, v, rows=rows).reshape(len(rows), Hq * D)

    h1 = h[rows] + attn @ _f64(w.w_o).T
    u2 = rms_norm(h1, w.ln_post, dims.rms_eps)
    act = silu(u2 @ _f64(w.w_gate).T) * (u2 @ _f64(w.w_up).T)
    return h1 + act @ _f64(w.w_down).T


def deepstack_add(h, visual_mask, feature) -> np.ndarray:
    """Add one DeepStack level's features to the visual-token rows.

    H3 encoder page, ``MiniMaxH3Qwen3VLTextModel._deepstack_process``: the
    rows of h selected by the boolean mask (in ascending token order) get the
    feature rows added, row r of the feature going to the r-th selected token.
    """
    out = _f64(h).copy()
    idx = np.flatnonzero(np.asarray(visual_mask, dtype=bool))
    feature = _f64(feature)
    if feature.shape[0] != idx.size:
        raise ValueError(f"{feature.shape[0]} feature rows for {idx.size} visual tokens")
    out[idx] += feature
    return out


def encode(embeds, positions, layers, dims: ModelDims, visual_mask=None,
           deepstack: Optional[Sequence[np.ndarray]] = None,
           n_layers: Optional[int] = None, return_all: bool = False):
    """Unnormalised hidden state after ``n_layers`` decoder layers.

    H3 encoder page, ``MiniMaxH3Qwen3VLTextModel.forward``: the rotary
    tables are built once from the [3, S] positions; each layer is applied in
    turn and, after layer l with l < len(deepstack), DeepStack level l is added
    to the visual rows. There is no final norm (the page keeps only the first
    layers and returns hidden_states[n_layers]).

    ``layers`` is a sequence of ``LayerWeights`` or a callable ``l -> LayerWeights``
    (so large stacks can be regenerated layer by layer). With ``return_all``
    the list [hidden_states[0], ..., hidden_states[n_layers]] is returned.
    """
    h = _f64(embeds)
    if n_layers is None:
        n_layers = len(layers)
    cos, sin = rope_cos_sin(positions, dims.head_dim, dims.rope_theta, dims.mrope_section)
    states = [h] if return_all else None
    n_ds = 0 if deepstack is None else len(deepstack)
    for l in range(n_layers):
        w = layers(l) if callable(layers) else layers[l]
        h = decoder_layer(h, w, cos, sin, dims)
        if l < n_ds:
            h = deepstack_add(h, visual_mask, deepstack[l])
        if return_all:
            states.append(h)
    return states if return_all else h


def layer_param_count(dims: ModelDims) -> int:
    """Weight parameters of one decoder layer (linear weights plus the four gains)."""
    H, D, Hq, Hkv, I = dims.hidden, dims.head_dim, dims.n_heads, dims.n_kv_heads, dims.intermediate
    linear = (Hq + 2 * Hkv) * D * H + H * Hq * D + 2 * I * H + H * I
    gains = 2 * H + 2 * D
    return linear + gains
