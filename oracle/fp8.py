"""Online FP8 variant of the decoder's linear layers, as plain reference code.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

H3 encoder page: the encoder accepts an FP8 quantisation config only when the
checkpoint is not FP8-serialised (``_validate_encoder_quant_config``), i.e.
weights are quantised when loaded, and every linear layer then runs through
its quantised method (``_is_quantized_linear`` selects the fused qkv and
gate/up GEMMs). The page does not print the method itself; the reading taken
here is the plain per-tensor one:

* FP8 is OCP E4M3 (the "fn" variant: 4 exponent bits with bias 7, 3 mantissa
  bits, no infinities, largest finite 448);
* a tensor x is quantised with one scale s = max|x| / 448 as
  q = E4M3(round-to-nearest-even(clip(x * (448 / max|x|), -448, 448))), the
  factor and the product taken in float32 (the precision of the kernel that
  decides the code); the weights once, each activation on every call;
* the tensors are those of the page's linear layers: the fused qkv weight
  (q, k and v rows stacked) and the fused gate_up weight (gate rows, then up
  rows) are one tensor each, with one scale, like the o and down weights;
* y = (q_x q_w^T) * s_x * s_w, accumulated exactly (here float64), before
  the layer's bias / residual / SiLU epilogue.

Everything else of the decoder layer is unchanged (``qwen3vl_text``).
"""

from __future__ import annotations

import numpy as np

from .qwen3vl_text import (LayerWeights, ModelDims, apply_rope, causal_gqa_attention,
                           rms_norm, silu)

E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """The 256 codes of E4M3 (fn) decoded (NaN for 0x7f and 0xff)."""
    out = np.empty(256)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = sign * m * 2.0 ** -9          # subnormals: m/8 * 2^-6
        else:
            out[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def round_e4m3(x) -> np.ndarray:
    """Round to the nearest finite E4M3 value, ties to the even mantissa;
    |x| must be <= 448 (callers clip first).

    A magnitude in the binade [2^E, 2^(E+1)) lies on a grid of step
    2^(E-3) (3 mantissa bits); below 2^-6 the subnormal step 2^-9 holds. So
    the value is its magnitude divided by that step, rounded half to even,
    times the step (all exact in float64)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > E4M3_MAX):
        raise ValueError("value beyond the E4M3 range")
    _, e = np.frexp(a)                                   # a = m 2^e, m in [0.5, 1)
    step = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    r = np.round(a / step) * step                        # np.round: half to even
    return np.where(x < 0, -r, r)


def tensor_scale(x):
    """(float32 factor 448 / max|x|, scale s = max|x| / 448) of a whole tensor;
    (None, 1.0) for an all-zero tensor."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    if amax == 0:
        return None, 1.0
    return np.float32(E4M3_MAX) / amax, float(amax) / E4M3_MAX


def codes(x, factor):
    """The E4M3 values of x under a tensor's float32 factor: x * factor in
    float32, clipped to +-448, rounded to the grid (zeros when factor is None)."""
    x32 = np.asarray(x, dtype=np.float32)
    if factor is None:
        return np.zeros(x32.shape)
    y = np.clip(x32 * factor, -E4M3_MAX, E4M3_MAX).astype(np.float64)
    return round_e4m3(y)


def quantize(x, threads: int = 1):
    """(q as float64 values on the E4M3 grid, scale s) of the per-tensor scheme.

    Every code depends on its own element and the tensor's factor only, so
    with threads > 1 the codes of separate row blocks are formed on a thread
    pool (NumPy's element-wise loops release the interpreter lock); the
    values are the same."""
    factor, scale = tensor_scale(x)
    x = np.asarray(x)
    if threads <= 1 or x.ndim < 2 or x.shape[0] < 2 * threads:
        return codes(x, factor), scale
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty(x.shape)
    bounds = np.linspace(0, x.shape[0], 4 * threads + 1).astype(int)

    def one(i):
        out[bounds[i]:bounds[i + 1]] = codes(x[bounds[i]:bounds[i + 1]], factor)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(len(bounds) - 1)))
    return out, scale


def linear_fp8(x, w_q, w_scale, threads: int = 1):
    """x (float) quantised on the fly times an already-quantised weight."""
    q_x, s_x = quantize(x, threads)
    return (q_x @ np.asarray(w_q, dtype=np.float64).T) * (s_x * w_scale)


# the page's linear layers and the weight rows each one stacks
FUSED = {"w_qkv": ("w_q", "w_k", "w_v"), "w_o": ("w_o",), "w_gate_up": ("w_gate", "w_up"),
         "w_down": ("w_down",)}


def quantize_layer(w: LayerWeights, threads: int = 1):
    """Quantised weights of a layer: {linear: (values, scale)}, one scale per
    linear layer over its stacked rows."""
    return {name: quantize(np.concatenate([np.asarray(getattr(w, p), dtype=np.float64) for p in parts]),
                           threads)
            for name, parts in FUSED.items()}


def decoder_layer_fp8(h, w: LayerWeights, qw, cos, sin, dims: ModelDims, threads: int = 1):
    """The decoder layer with every linear in FP8 (qw from quantize_layer), all
    rows (the activation scales are taken over whole tensors). `threads`: as
    for quantize."""
    h = np.asarray(h, dtype=np.float64)
    S = h.shape[0]
    rows = np.arange(S)
    need = S
    D, Hq, Hkv = dims.head_dim, dims.n_heads, dims.n_kv_heads
    u = rms_norm(h[:need], w.ln_in, dims.rms_eps)
    qkv = linear_fp8(u, *qw["w_qkv"], threads)
    q = qkv[:, :Hq * D].reshape(need, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(need, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(need, Hkv, D)
    q = rms_norm(q, w.q_norm, dims.rms_eps)
    k = rms_norm(k, w.k_norm, dims.rms_eps)
    q = apply_rope(q, cos[:need], sin[:need])
    k = apply_rope(k, cos[:need], sin[:need])
    o = causal_gqa_attention(q, k, v, rows)
    x = h[rows] + linear_fp8(o.reshape(S, Hq * D), *qw["w_o"], threads)
    u2 = rms_norm(x, w.ln_post, dims.rms_eps)
    gu = linear_fp8(u2, *qw["w_gate_up"], threads)
    I = dims.intermediate
    return x + linear_fp8(silu(gu[:, :I]) * gu[:, I:], *qw["w_down"], threads)
