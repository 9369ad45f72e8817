"""ctypes binding of libmhe (the C ABI declared in ``include/mhe.h``).

Argument marshalling only: every function here forwards device pointers,
sizes and a HIP stream to the library of the same name, which does all of the
computation. Arguments may be torch tensors (their ``data_ptr()`` is passed)
or plain integers (raw device addresses). The stream defaults to torch's
current stream on the current device.

The library is loaded on first use; if ``libmhe.so`` has not been built the
call fails loudly (there is no fallback path).
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmhe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "mhe.h")

MHE_OK = 0
STATUS_NAMES = {0: "MHE_OK", 1: "MHE_ERR_NULL", 2: "MHE_ERR_SHAPE", 3: "MHE_ERR_MISMATCH",
                4: "MHE_ERR_UNSUPPORTED", 5: "MHE_ERR_WORKSPACE", 6: "MHE_ERR_HIP"}


class MheError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        self.fn, self.status, self.message = fn, status, message
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {message}")


class MheConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("mrope_section", ctypes.c_int32 * 3)]


WEIGHT_FIELDS = ("ln_in", "w_q", "w_k", "w_v", "q_norm", "k_norm", "w_o", "ln_post",
                 "w_gate", "w_up", "w_down")


class MheLayerWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in WEIGHT_FIELDS]


FP8_WEIGHT_FIELDS = (("ln_in", False), ("w_qkv", False), ("s_qkv", True), ("q_norm", False),
                     ("k_norm", False), ("w_o", False), ("s_o", True), ("ln_post", False),
                     ("w_gate_up", False), ("s_gate_up", True), ("w_down", False), ("s_down", True))


class MheLayerWeightsFp8(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name, _ in FP8_WEIGHT_FIELDS]


class MheVisionConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("depth", ctypes.c_int32),
                ("patch_dim", ctypes.c_int32), ("merge", ctypes.c_int32),
                ("out_hidden", ctypes.c_int32), ("pos_side", ctypes.c_int32),
                ("n_deepstack", ctypes.c_int32), ("deepstack_index", ctypes.c_int32 * 8)]


VISION_BLOCK_FIELDS = ("norm1_w", "norm1_b", "qkv_w", "qkv_b", "proj_w", "proj_b", "norm2_w",
                       "norm2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")
VISION_MERGER_FIELDS = ("norm_w", "norm_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")


class MheVisionBlockWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in VISION_BLOCK_FIELDS]


class MheVisionMergerWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in VISION_MERGER_FIELDS]


class MheVisionWeights(ctypes.Structure):
    _fields_ = [("patch_w", ctypes.c_void_p), ("patch_b", ctypes.c_void_p),
                ("pos_table", ctypes.c_void_p), ("blocks", ctypes.POINTER(MheVisionBlockWeights)),
                ("merger", MheVisionMergerWeights),
                ("deepstack", ctypes.POINTER(MheVisionMergerWeights))]


_lib: Optional[ctypes.CDLL] = None

_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_SIGNATURES = {
    "mhe_abi_version": (_i32, []),
    "mhe_status_string": (ctypes.c_char_p, [_i32]),
    "mhe_last_error": (ctypes.c_char_p, []),
    "mhe_workspace_bytes": (_sz, [ctypes.POINTER(MheConfig), _i32]),
    "mhe_layer_forward": (_i32, [ctypes.POINTER(MheConfig), ctypes.POINTER(MheLayerWeights), _vp,
                                 _vp, _i32, _vp, _sz, _vp]),
    "mhe_deepstack_inject": (_i32, [_vp, _i32, _i32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "mhe_deepstack_inject_noalloc": (_i32, [_vp, _i32, _i32, _vp, _i32, _vp, _vp]),
    "mhe_encode": (_i32, [ctypes.POINTER(MheConfig), ctypes.POINTER(MheLayerWeights), _i32, _vp,
                          _vp, _vp, _i32, ctypes.POINTER(_vp), _i32, _i32, _vp, _vp, _sz, _vp]),
    "mhe_count_visual": (_i32, [_vp, _i32, ctypes.POINTER(_i32), _vp, _sz, _vp]),
    "mhe_rms_norm": (_i32, [_vp, _vp, _vp, _i32, _i32, _f32, _vp]),
    "mhe_linear_workspace_bytes": (_sz, []),
    "mhe_linear": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "mhe_linear_swiglu": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "mhe_qk_norm_rope": (_i32, [ctypes.POINTER(MheConfig), _vp, _vp, _vp, _vp, _i32, _vp, _vp,
                                _vp, _vp]),
    "mhe_attention": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "mhe_qnorm_attention_workspace_bytes": (_sz, [ctypes.POINTER(MheConfig), _i32]),
    "mhe_qnorm_attention": (_i32, [ctypes.POINTER(MheConfig), _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]),
    "mhe_trace_enable": (_i32, [ctypes.c_uint32]),
    "mhe_trace_read": (_i32, [_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
    "mhe_rope_index": (_i32, [_vp, _i32, _i32, _i32, _vp, _i32, _vp, _i32, _i32, _vp, _vp, _vp,
                              _vp, ctypes.POINTER(_i32)]),
    "mhe_embed_tokens": (_i32, [_vp, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "mhe_scatter_visual": (_i32, [_vp, _i32, _i32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "mhe_join_visual_workspace_bytes": (_sz, [_i32]),
    "mhe_join_visual": (_i32, [_vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "mhe_vision_workspace_bytes": (_sz, [ctypes.POINTER(MheVisionConfig), _i32]),
    "mhe_vision_forward": (_i32, [ctypes.POINTER(MheVisionConfig), ctypes.POINTER(MheVisionWeights),
                                  _vp, _vp, _i32, _vp, ctypes.POINTER(_vp), _vp, _sz, _vp]),
    "mhe_vision_embed": (_i32, [ctypes.POINTER(MheVisionConfig), ctypes.POINTER(MheVisionWeights),
                                _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "mhe_vision_blocks": (_i32, [ctypes.POINTER(MheVisionConfig), ctypes.POINTER(MheVisionWeights),
                                 _i32, _i32, _vp, _vp, _i32, _vp, _sz, _vp]),
    "mhe_vision_merge": (_i32, [ctypes.POINTER(MheVisionConfig),
                                ctypes.POINTER(MheVisionMergerWeights), _i32, _vp, _i32, _vp, _vp,
                                _sz, _vp]),
    "mhe_layer_norm": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _f32, _vp]),
    "mhe_quantize_fp8_workspace_bytes": (_sz, []),
    "mhe_quantize_fp8": (_i32, [ctypes.POINTER(_vp), ctypes.POINTER(_i32), _i32, _i32, _vp, _vp,
                                _vp, _sz, _vp]),
    "mhe_linear_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "mhe_linear_swiglu_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "mhe_workspace_bytes_fp8": (_sz, [ctypes.POINTER(MheConfig), _i32]),
    "mhe_layer_forward_fp8": (_i32, [ctypes.POINTER(MheConfig), ctypes.POINTER(MheLayerWeightsFp8),
                                     _vp, _vp, _i32, _vp, _sz, _vp]),
    "mhe_encode_fp8": (_i32, [ctypes.POINTER(MheConfig), ctypes.POINTER(MheLayerWeightsFp8), _i32,
                              _vp, _vp, _vp, _i32, ctypes.POINTER(_vp), _i32, _i32, _vp, _vp, _sz,
                              _vp]),
    "mhe_linear_bias": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz, _vp]),
    "mhe_vision_attention_workspace_bytes": (_sz, [_i32]),
    "mhe_vision_attention": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _i32, _vp, _sz,
                                    _vp]),
}

# placeholder token ids of Qwen3-VL (H3 encoder page, MiniMaxH3Qwen3VLEncoder defaults)
IMAGE_TOKEN_ID = 151655
VIDEO_TOKEN_ID = 151656

# step ids of the trace facility (MHE_STEP_* in include/mhe.h)
STEPS = ("input_norm", "qkv", "qk_rope", "attention", "o_proj", "post_norm", "gate_up", "down",
         "deepstack", "quantize")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m multimodal_encoder_prefill_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def header_entry_points() -> list:
    """Names of the functions that include/mhe.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhe_[a-z0-9_]+)\s*\(", text)))


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != MHE_OK:
        msg = lib().mhe_last_error().decode(errors="replace")
        raise MheError(fn, rc, msg)


def make_config(hidden, n_heads, n_kv_heads, head_dim, intermediate, rms_eps=1e-6,
                rope_theta=5e6, mrope_section=(24, 20, 20)) -> MheConfig:
    c = MheConfig()
    c.hidden, c.n_heads, c.n_kv_heads, c.head_dim = hidden, n_heads, n_kv_heads, head_dim
    c.intermediate, c.rms_eps, c.rope_theta = intermediate, rms_eps, rope_theta
    for i in range(3):
        c.mrope_section[i] = int(mrope_section[i])
    return c


def config_from_dims(d) -> MheConfig:
    return make_config(d.hidden, d.n_heads, d.n_kv_heads, d.head_dim, d.intermediate,
                       d.rms_eps, d.rope_theta, d.mrope_section)


def layer_table(weights) -> MheLayerWeights:
    """Weight table from a mapping name -> tensor (or device address)."""
    t = MheLayerWeights()
    for name in WEIGHT_FIELDS:
        setattr(t, name, _ptr(weights[name]))
    return t


def abi_version() -> int:
    return lib().mhe_abi_version()


def status_string(status: int) -> str:
    return lib().mhe_status_string(status).decode()


def workspace_bytes(cfg: MheConfig, seq: int) -> int:
    n = lib().mhe_workspace_bytes(ctypes.byref(cfg), seq)
    if n == 0:
        raise MheError("mhe_workspace_bytes", 2, lib().mhe_last_error().decode())
    return n


def layer_forward(cfg, weights, hidden, positions, seq, workspace, workspace_bytes, stream=None):
    table = weights if isinstance(weights, MheLayerWeights) else layer_table(weights)
    _check("mhe_layer_forward", lib().mhe_layer_forward(
        ctypes.byref(cfg), ctypes.byref(table), _ptr(hidden), _ptr(positions), seq,
        _ptr(workspace), workspace_bytes, _stream(stream)))


def deepstack_inject(hidden, seq, hidden_dim, visual_mask, n_vis, feature, workspace,
                     workspace_bytes, stream=None):
    _check("mhe_deepstack_inject", lib().mhe_deepstack_inject(
        _ptr(hidden), seq, hidden_dim, _ptr(visual_mask), n_vis, _ptr(feature),
        _ptr(workspace), workspace_bytes, _stream(stream)))


def deepstack_inject_noalloc(hidden, seq, hidden_dim, visual_mask, n_vis, feature, stream=None):
    _check("mhe_deepstack_inject_noalloc", lib().mhe_deepstack_inject_noalloc(
        _ptr(hidden), seq, hidden_dim, _ptr(visual_mask), n_vis, _ptr(feature), _stream(stream)))


def encode(cfg, layers: Sequence, inputs_embeds, positions, seq, out, workspace,
           workspace_bytes, visual_mask=None, n_vis=0, deepstack: Optional[Sequence] = None,
           stream=None):
    n_layers = len(layers)
    tables = (MheLayerWeights * max(n_layers, 1))()
    for i, w in enumerate(layers):
        tables[i] = w if isinstance(w, MheLayerWeights) else layer_table(w)
    n_ds = 0 if deepstack is None else len(deepstack)
    ds = (ctypes.c_void_p * max(n_ds, 1))()
    for i in range(n_ds):
        ds[i] = _ptr(deepstack[i])
    _check("mhe_encode", lib().mhe_encode(
        ctypes.byref(cfg), tables if n_layers else None, n_layers, _ptr(inputs_embeds),
        _ptr(positions), _ptr(visual_mask), n_vis, ds if n_ds else None, n_ds, seq, _ptr(out),
        _ptr(workspace), workspace_bytes, _stream(stream)))


def count_visual(visual_mask, seq, workspace, workspace_bytes, stream=None) -> int:
    n = ctypes.c_int32(-1)
    _check("mhe_count_visual", lib().mhe_count_visual(
        _ptr(visual_mask), seq, ctypes.byref(n), _ptr(workspace), workspace_bytes,
        _stream(stream)))
    return n.value


def rms_norm(x, gamma, y, rows, dim, eps, stream=None):
    _check("mhe_rms_norm", lib().mhe_rms_norm(_ptr(x), _ptr(gamma), _ptr(y), rows, dim, eps,
                                              _stream(stream)))


def linear_workspace_bytes() -> int:
    return lib().mhe_linear_workspace_bytes()


def _ws(workspace):
    if workspace is None:
        return None, 0
    if isinstance(workspace, tuple):
        return workspace
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def linear(a, w, c, m, n, k, residual=None, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check("mhe_linear", lib().mhe_linear(_ptr(a), _ptr(w), _ptr(c), _ptr(residual), m, n, k,
                                          wp, wb, _stream(stream)))


def linear_swiglu(a, w_gate, w_up, c, m, n, k, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check("mhe_linear_swiglu", lib().mhe_linear_swiglu(_ptr(a), _ptr(w_gate), _ptr(w_up),
                                                        _ptr(c), m, n, k, wp, wb, _stream(stream)))


# ---- FP8 linears ----

def quantize_fp8_workspace_bytes() -> int:
    return lib().mhe_quantize_fp8_workspace_bytes()


def quantize_fp8(parts: Sequence, part_rows: Sequence[int], cols, q, scale, workspace, stream=None):
    """One per-tensor E4M3 quantisation of the row blocks `parts` (stacked in q)."""
    n = len(parts)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[_ptr(p) for p in parts])
    rows = (ctypes.c_int32 * max(n, 1))(*[int(r) for r in part_rows])
    wp, wb = _ws(workspace)
    _check("mhe_quantize_fp8", lib().mhe_quantize_fp8(ptrs, rows, n, cols, _ptr(q), _ptr(scale),
                                                      wp, wb, _stream(stream)))


def linear_fp8(a, scale_a, w, scale_w, c, m, n, k, residual=None, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check("mhe_linear_fp8", lib().mhe_linear_fp8(_ptr(a), _ptr(scale_a), _ptr(w), _ptr(scale_w),
                                                  _ptr(c), _ptr(residual), m, n, k, wp, wb,
                                                  _stream(stream)))


def linear_swiglu_fp8(a, scale_a, w_gate_up, scale_w, c, m, n, k, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check("mhe_linear_swiglu_fp8", lib().mhe_linear_swiglu_fp8(
        _ptr(a), _ptr(scale_a), _ptr(w_gate_up), _ptr(scale_w), _ptr(c), m, n, k, wp, wb,
        _stream(stream)))


def layer_table_fp8(weights) -> MheLayerWeightsFp8:
    """FP8 weight table from a mapping name -> tensor (or device address)."""
    t = MheLayerWeightsFp8()
    for name, _ in FP8_WEIGHT_FIELDS:
        setattr(t, name, _ptr(weights[name]))
    return t


def workspace_bytes_fp8(cfg: MheConfig, seq: int) -> int:
    n = lib().mhe_workspace_bytes_fp8(ctypes.byref(cfg), seq)
    if n == 0:
        raise MheError("mhe_workspace_bytes_fp8", 2, lib().mhe_last_error().decode())
    return n


def layer_forward_fp8(cfg, weights, hidden, positions, seq, workspace, workspace_bytes, stream=None):
    table = weights if isinstance(weights, MheLayerWeightsFp8) else layer_table_fp8(weights)
    _check("mhe_layer_forward_fp8", lib().mhe_layer_forward_fp8(
        ctypes.byref(cfg), ctypes.byref(table), _ptr(hidden), _ptr(positions), seq,
        _ptr(workspace), workspace_bytes, _stream(stream)))


def encode_fp8(cfg, layers: Sequence, inputs_embeds, positions, seq, out, workspace,
               workspace_bytes, visual_mask=None, n_vis=0, deepstack: Optional[Sequence] = None,
               stream=None):
    n_layers = len(layers)
    tables = (MheLayerWeightsFp8 * max(n_layers, 1))()
    for i, w in enumerate(layers):
        tables[i] = w if isinstance(w, MheLayerWeightsFp8) else layer_table_fp8(w)
    n_ds = 0 if deepstack is None else len(deepstack)
    ds = (ctypes.c_void_p * max(n_ds, 1))()
    for i in range(n_ds):
        ds[i] = _ptr(deepstack[i])
    _check("mhe_encode_fp8", lib().mhe_encode_fp8(
        ctypes.byref(cfg), tables if n_layers else None, n_layers, _ptr(inputs_embeds),
        _ptr(positions), _ptr(visual_mask), n_vis, ds if n_ds else None, n_ds, seq, _ptr(out),
        _ptr(workspace), workspace_bytes, _stream(stream)))


class Fp8Layer:
    """Device buffers of one decoder layer quantised for the FP8 forms: the
    fused qkv and gate_up weights and the o and down weights as E4M3 tensors
    with one scale each (mhe_quantize_fp8), the norms shared with the bf16
    weights. `weights`: name -> bf16 device tensor as for layer_table."""

    def __init__(self, weights, cfg: MheConfig, stream=None):
        import torch
        dev = weights["w_q"].device
        H, I = cfg.hidden, cfg.intermediate
        qw, kvw = cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
        ws = torch.empty(quantize_fp8_workspace_bytes(), dtype=torch.uint8, device=dev)
        self.tensors = {}
        for name, parts, rows, cols in (
                ("w_qkv", ("w_q", "w_k", "w_v"), (qw, kvw, kvw), H),
                ("w_o", ("w_o",), (H,), qw),
                ("w_gate_up", ("w_gate", "w_up"), (I, I), H),
                ("w_down", ("w_down",), (H,), I)):
            q = torch.empty((sum(rows), cols), dtype=torch.uint8, device=dev)
            s = torch.empty(1, dtype=torch.float32, device=dev)
            quantize_fp8([weights[p] for p in parts], rows, cols, q, s, ws, stream)
            self.tensors[name] = q
            self.tensors["s_" + name[2:]] = s
        for name in ("ln_in", "q_norm", "k_norm", "ln_post"):
            self.tensors[name] = weights[name]
        torch.cuda.synchronize(dev)  # before the quantisation workspace is released
        self.table = layer_table_fp8(self.tensors)


def qk_norm_rope(cfg, qkv, q_norm, k_norm, positions, seq, q_out, k_out, vt_out, stream=None):
    _check("mhe_qk_norm_rope", lib().mhe_qk_norm_rope(
        ctypes.byref(cfg), _ptr(qkv), _ptr(q_norm), _ptr(k_norm), _ptr(positions), seq,
        _ptr(q_out), _ptr(k_out), _ptr(vt_out), _stream(stream)))


def attention(q, k, vt, o, seq, n_heads, n_kv_heads, head_dim, stream=None):
    _check("mhe_attention", lib().mhe_attention(_ptr(q), _ptr(k), _ptr(vt), _ptr(o), seq,
                                                n_heads, n_kv_heads, head_dim, _stream(stream)))


def qnorm_attention_workspace_bytes(cfg, seq) -> int:
    return int(lib().mhe_qnorm_attention_workspace_bytes(ctypes.byref(cfg), seq))


def qnorm_attention(cfg, qkv, q_norm, positions, k, vt, o, seq, workspace, workspace_bytes, stream=None):
    _check("mhe_qnorm_attention", lib().mhe_qnorm_attention(
        ctypes.byref(cfg), _ptr(qkv), _ptr(q_norm), _ptr(positions), _ptr(k), _ptr(vt), _ptr(o), seq,
        _ptr(workspace), workspace_bytes, _stream(stream)))


def trace_enable(steps) -> None:
    """Record launch times of the named steps (an iterable of STEPS names; empty = off)."""
    mask = 0
    for name in steps:
        mask |= 1 << STEPS.index(name)
    _check("mhe_trace_enable", lib().mhe_trace_enable(mask))


def trace_read(step: str):
    """(total milliseconds, launches) recorded for `step` since the last read."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check("mhe_trace_read", lib().mhe_trace_read(STEPS.index(step), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def seq_pad(seq: int) -> int:
    """Padded token count of the K / V^T layouts (multiple of 128)."""
    return (seq + 127) // 128 * 128


# ---- token-level front end ----

def rope_index(ids, image_token_id=IMAGE_TOKEN_ID, video_token_id=VIDEO_TOKEN_ID,
               image_grid_thw=None, video_grid_thw=None, spatial_merge=2):
    """Host call: (positions int32 [3, S], image_mask, video_mask, visual_mask uint8 [S], delta).

    ids: host token ids (sequence, numpy array or CPU tensor); grids: [n, 3] (t, h, w).
    """
    import numpy as np
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    seq = int(ids.shape[0])
    ig = np.ascontiguousarray(np.asarray(image_grid_thw if image_grid_thw is not None else
                                         np.zeros((0, 3)), dtype=np.int32).reshape(-1, 3))
    vg = np.ascontiguousarray(np.asarray(video_grid_thw if video_grid_thw is not None else
                                         np.zeros((0, 3)), dtype=np.int32).reshape(-1, 3))
    pos = np.empty((3, max(seq, 1)), dtype=np.int32)
    masks = [np.empty(max(seq, 1), dtype=np.uint8) for _ in range(3)]
    delta = ctypes.c_int32(0)
    _check("mhe_rope_index", lib().mhe_rope_index(
        ids.ctypes.data, seq, image_token_id, video_token_id,
        ig.ctypes.data if len(ig) else None, len(ig), vg.ctypes.data if len(vg) else None, len(vg),
        spatial_merge, pos.ctypes.data, masks[0].ctypes.data, masks[1].ctypes.data,
        masks[2].ctypes.data, ctypes.byref(delta)))
    return pos, masks[0], masks[1], masks[2], delta.value


def embed_tokens(ids, seq, table, row_begin, rows, hidden_dim, out, n_outside=None, stream=None):
    _check("mhe_embed_tokens", lib().mhe_embed_tokens(
        _ptr(ids), seq, _ptr(table), row_begin, rows, hidden_dim, _ptr(out), _ptr(n_outside),
        _stream(stream)))


def scatter_visual(hidden, seq, hidden_dim, mask, n, feature, workspace, workspace_bytes,
                   stream=None):
    _check("mhe_scatter_visual", lib().mhe_scatter_visual(
        _ptr(hidden), seq, hidden_dim, _ptr(mask), n, _ptr(feature), _ptr(workspace),
        workspace_bytes, _stream(stream)))


def join_visual_workspace_bytes(seq: int) -> int:
    return lib().mhe_join_visual_workspace_bytes(seq)


def join_visual(image_mask, video_mask, seq, hidden_dim, image_feature, n_image, video_feature,
                n_video, joint, workspace, workspace_bytes, stream=None):
    _check("mhe_join_visual", lib().mhe_join_visual(
        _ptr(image_mask), _ptr(video_mask), seq, hidden_dim, _ptr(image_feature), n_image,
        _ptr(video_feature), n_video, _ptr(joint), _ptr(workspace), workspace_bytes,
        _stream(stream)))


def encode_ids(cfg, layers: Sequence, ids, embed_table, out, workspace, workspace_bytes, *,
               image_embeds=None, image_grid_thw=None, video_embeds=None, video_grid_thw=None,
               deepstack_image: Optional[Sequence] = None,
               deepstack_video: Optional[Sequence] = None,
               image_token_id=IMAGE_TOKEN_ID, video_token_id=VIDEO_TOKEN_ID, spatial_merge=2,
               stream=None):
    """The page's encode_ids from token ids and vision-tower outputs, as libmhe calls.

    ids: host token ids [S]; embed_table device bf16 [vocab, hidden]; image / video
    embeds device bf16 [n, hidden] (rows in placeholder order) with their grids;
    deepstack_* lists of device bf16 [n, hidden] per level. `out` [S, hidden] receives
    the layer output. Raises ValueError when feature and placeholder counts differ
    (H3 encoder page, _get_placeholder_mask).
    """
    import numpy as np
    import torch
    pos, img_m, vid_m, vis_m, _ = rope_index(ids, image_token_id, video_token_id,
                                             image_grid_thw, video_grid_thw, spatial_merge)
    seq = pos.shape[1] if len(np.asarray(ids)) else 0
    n_img, n_vid = int(img_m[:seq].sum()), int(vid_m[:seq].sum())
    for name, feats, n in (("image", image_embeds, n_img), ("video", video_embeds, n_vid)):
        if feats is not None and feats.shape[0] != n:
            raise ValueError(f"{name} features and tokens do not match: tokens {n}, features {feats.shape[0]}")
    dev = out.device
    hidden = cfg.hidden
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a[..., :seq])).to(dev)
    ids_dev = up(np.asarray(ids, dtype=np.int32))
    pos_dev, img_dev, vid_dev, vis_dev = up(pos), up(img_m), up(vid_m), up(vis_m)
    embeds = torch.empty(seq, hidden, dtype=torch.bfloat16, device=dev)
    embed_tokens(ids_dev, seq, embed_table, 0, embed_table.shape[0], hidden, embeds, stream=stream)
    small = torch.empty(join_visual_workspace_bytes(seq), dtype=torch.uint8, device=dev)
    nb = small.numel()
    if image_embeds is not None:
        scatter_visual(embeds, seq, hidden, img_dev, n_img, image_embeds, small, nb, stream)
    if video_embeds is not None:
        scatter_visual(embeds, seq, hidden, vid_dev, n_vid, video_embeds, small, nb, stream)
    # DeepStack rows in token order over every visual token (_aggregate_deepstack)
    levels, mask, n_vis = None, None, 0
    if deepstack_image is not None and deepstack_video is not None:
        levels = []
        for di, dv in zip(deepstack_image, deepstack_video):
            joint = torch.empty(n_img + n_vid, hidden, dtype=torch.bfloat16, device=dev)
            join_visual(img_dev, vid_dev, seq, hidden, di, n_img, dv, n_vid, joint, small, nb,
                        stream)
            levels.append(joint)
        mask, n_vis = vis_dev, n_img + n_vid
    elif deepstack_image is not None:
        levels, mask, n_vis = list(deepstack_image), img_dev, n_img
    elif deepstack_video is not None:
        levels, mask, n_vis = list(deepstack_video), vid_dev, n_vid
    encode(cfg, layers, embeds, pos_dev, seq, out, workspace, workspace_bytes,
           visual_mask=mask, n_vis=n_vis, deepstack=levels, stream=stream)
    return pos


# ---- vision tower ----

def vision_config(vd) -> MheVisionConfig:
    """From an object with hidden, n_heads, intermediate (stored width), depth,
    patch_dim, merge, out_hidden, pos_side, deepstack (synth.VisionDims)."""
    c = MheVisionConfig()
    c.hidden, c.n_heads, c.intermediate, c.depth = vd.hidden, vd.n_heads, vd.intermediate, vd.depth
    c.patch_dim, c.merge, c.out_hidden, c.pos_side = vd.patch_dim, vd.merge, vd.out_hidden, vd.pos_side
    c.n_deepstack = len(vd.deepstack)
    for i, d in enumerate(vd.deepstack):
        c.deepstack_index[i] = d
    return c


def _merger_table(m) -> MheVisionMergerWeights:
    t = MheVisionMergerWeights()
    for f in VISION_MERGER_FIELDS:
        setattr(t, f, _ptr(m[f]))
    return t


class VisionTables:
    """Host tables of a tower's device weights (dict as synth.vision_weights returns);
    keeps the ctypes arrays alive for the calls that use them."""

    def __init__(self, w):
        self.blocks = (MheVisionBlockWeights * max(len(w["blocks"]), 1))()
        for i, b in enumerate(w["blocks"]):
            for f in VISION_BLOCK_FIELDS:
                setattr(self.blocks[i], f, _ptr(b[f]))
        self.ds = (MheVisionMergerWeights * max(len(w["deepstack"]), 1))()
        for i, m in enumerate(w["deepstack"]):
            self.ds[i] = _merger_table(m)
        self.merger = _merger_table(w["merger"])
        self.table = MheVisionWeights()
        self.table.patch_w, self.table.patch_b = _ptr(w["patch_w"]), _ptr(w["patch_b"])
        self.table.pos_table = _ptr(w["pos_table"])
        self.table.blocks = ctypes.cast(self.blocks, ctypes.POINTER(MheVisionBlockWeights))
        self.table.merger = self.merger
        self.table.deepstack = ctypes.cast(self.ds, ctypes.POINTER(MheVisionMergerWeights))


def _grids(grid_thw):
    import numpy as np
    g = np.ascontiguousarray(np.asarray(grid_thw, dtype=np.int32).reshape(-1, 3))
    return g, len(g)


def vision_workspace_bytes(cfg: MheVisionConfig, n_patches: int) -> int:
    n = lib().mhe_vision_workspace_bytes(ctypes.byref(cfg), n_patches)
    if n == 0:
        raise MheError("mhe_vision_workspace_bytes", 2, lib().mhe_last_error().decode())
    return n


def vision_forward(cfg, tables: VisionTables, pixels, grid_thw, merged, deepstack, workspace,
                   workspace_bytes, stream=None):
    g, ng = _grids(grid_thw)
    ds = (ctypes.c_void_p * max(len(deepstack), 1))(*[_ptr(d) for d in deepstack])
    _check("mhe_vision_forward", lib().mhe_vision_forward(
        ctypes.byref(cfg), ctypes.byref(tables.table), _ptr(pixels), g.ctypes.data, ng,
        _ptr(merged), ds, _ptr(workspace), workspace_bytes, _stream(stream)))


def vision_embed(cfg, tables: VisionTables, pixels, grid_thw, hidden, workspace, workspace_bytes,
                 stream=None):
    g, ng = _grids(grid_thw)
    _check("mhe_vision_embed", lib().mhe_vision_embed(
        ctypes.byref(cfg), ctypes.byref(tables.table), _ptr(pixels), g.ctypes.data, ng,
        _ptr(hidden), _ptr(workspace), workspace_bytes, _stream(stream)))


def vision_blocks(cfg, tables: VisionTables, first, count, hidden, grid_thw, workspace,
                  workspace_bytes, stream=None):
    g, ng = _grids(grid_thw)
    _check("mhe_vision_blocks", lib().mhe_vision_blocks(
        ctypes.byref(cfg), ctypes.byref(tables.table), first, count, _ptr(hidden), g.ctypes.data,
        ng, _ptr(workspace), workspace_bytes, _stream(stream)))


def vision_merge(cfg, merger, postshuffle, hidden, n_patches, out, workspace, workspace_bytes,
                 stream=None):
    t = merger if isinstance(merger, MheVisionMergerWeights) else _merger_table(merger)
    _check("mhe_vision_merge", lib().mhe_vision_merge(
        ctypes.byref(cfg), ctypes.byref(t), int(bool(postshuffle)), _ptr(hidden), n_patches,
        _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)))


def layer_norm(x, w, b, y, rows, dim, eps=1e-6, stream=None):
    _check("mhe_layer_norm", lib().mhe_layer_norm(_ptr(x), _ptr(w), _ptr(b), _ptr(y), rows, dim,
                                                  eps, _stream(stream)))


def linear_bias(a, w, bias, c, m, n, k, act=0, residual=None, workspace=None, stream=None):
    """act: 0 none, 1 GELU (tanh form), 2 GELU (erf form)."""
    wp, wb = _ws(workspace)
    _check("mhe_linear_bias", lib().mhe_linear_bias(_ptr(a), _ptr(w), _ptr(bias), _ptr(c),
                                                    _ptr(residual), m, n, k, act, wp, wb,
                                                    _stream(stream)))


def vision_attention_workspace_bytes(n_patches: int) -> int:
    n = lib().mhe_vision_attention_workspace_bytes(n_patches)
    if n == 0:
        raise MheError("mhe_vision_attention_workspace_bytes", 2, lib().mhe_last_error().decode())
    return n


def vision_attention(q, k, vt, o, n_patches, n_heads, head_dim, grid_thw, merge, workspace,
                     workspace_bytes, stream=None):
    g, ng = _grids(grid_thw)
    _check("mhe_vision_attention", lib().mhe_vision_attention(
        _ptr(q), _ptr(k), _ptr(vt), _ptr(o), n_patches, n_heads, head_dim, g.ctypes.data, ng,
        merge, _ptr(workspace), workspace_bytes, _stream(stream)))
