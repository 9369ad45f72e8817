"""The C-ABI library loads, exports every declared entry point and rejects bad
arguments on the host before any launch (no GPU needed: every call here fails
validation, so nothing reaches the HIP runtime)."""

import ctypes

import pytest

from multimodal_encoder_prefill_amd import binding as b
from multimodal_encoder_prefill_amd import synth


def test_every_declared_symbol_is_exported():
    names = b.header_entry_points()
    assert len(names) >= 13
    lib = b.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(b._SIGNATURES)


def test_status_strings_and_version():
    assert b.abi_version() == 1
    assert b.status_string(0) == "ok"
    assert "workspace" in b.status_string(5)


def test_workspace_bytes_scales_and_validates():
    cfg = b.config_from_dims(synth.FULL)
    part = b.linear_workspace_bytes()          # fixed split-K scratch
    w1 = b.workspace_bytes(cfg, 512)
    w2 = b.workspace_bytes(cfg, 4096)
    assert w2 - part > 7 * (w1 - part)
    # hidden + max(attention buffers: q|k|v, K, V^T, attention output; MLP
    # activation) + index list, 256-byte aligned pieces
    S = 4096
    attn = S * 10240 * 2 + 2 * 8 * 4096 * 128 * 2 + S * 8192 * 2
    assert w2 >= S * 5120 * 2 + max(attn, S * 25600 * 2) + S * 4 + part
    with pytest.raises(b.MheError):
        b.workspace_bytes(cfg, 0)
    bad = b.config_from_dims(synth.FULL)
    bad.n_kv_heads = 3
    with pytest.raises(b.MheError) as e:
        b.workspace_bytes(bad, 16)
    assert e.value.status == 2


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, 4), ("n_kv_heads", 1, 4), ("hidden", 100, 4), ("intermediate", 1000, 4),
    ("rope_theta", -1.0, 2), ("n_heads", 0, 2),
])
def test_config_rejections(field, value, status):
    cfg = b.config_from_dims(synth.FULL)
    setattr(cfg, field, value)
    rc = b.lib().mhe_workspace_bytes(ctypes.byref(cfg), 64)
    assert rc == 0
    assert b.lib().mhe_last_error()


def _layer_call(**over):
    cfg = b.config_from_dims(synth.TINY)
    table = b.MheLayerWeights(*([0x1000] * 11))
    args = dict(cfg=ctypes.byref(cfg), w=ctypes.byref(table), hidden=0x2000, pos=0x3000, seq=64,
                ws=0x10000, ws_bytes=1 << 40, stream=None)
    args.update(over)
    return b.lib().mhe_layer_forward(args["cfg"], args["w"], args["hidden"], args["pos"],
                                     args["seq"], args["ws"], args["ws_bytes"], args["stream"])


def test_layer_forward_rejects_before_launch():
    assert _layer_call(hidden=None) == 1
    assert _layer_call(pos=None) == 1
    assert _layer_call(seq=0) == 2
    assert _layer_call(ws_bytes=1024) == 5
    assert _layer_call(ws=0x10010) == 5          # misaligned
    assert _layer_call(w=None) == 1
    t = b.MheLayerWeights(*([0x1000] * 11))
    t.w_down = None
    assert _layer_call(w=ctypes.byref(t)) == 1
    assert "w_down" in b.lib().mhe_last_error().decode()
    t.w_down = 0x1008                             # not on a 16-byte boundary
    assert _layer_call(w=ctypes.byref(t)) == 2
    assert "w_down" in b.lib().mhe_last_error().decode()
    assert _layer_call(hidden=0x2004) == 2


def test_encode_rejects_before_launch():
    cfg = b.config_from_dims(synth.TINY)
    lib = b.lib()
    tables = (b.MheLayerWeights * 2)(b.MheLayerWeights(*([0x1000] * 11)), b.MheLayerWeights(*([0x1000] * 11)))
    ds = (ctypes.c_void_p * 1)(0x5000)
    call = lambda **o: lib.mhe_encode(ctypes.byref(cfg), o.get("layers", tables), o.get("n_layers", 2),
                                      o.get("emb", 0x2000), 0x3000, o.get("mask", 0x4000),
                                      o.get("n_vis", 8), o.get("ds", ds), o.get("n_ds", 1),
                                      o.get("seq", 64), o.get("out", 0x100000), 0x200000,
                                      o.get("ws_bytes", 1 << 30), None)
    assert call(n_vis=65) == 2               # more visual tokens than seq
    assert call(mask=None) == 1              # DeepStack without a mask
    assert call(ds=None) == 1
    assert call(n_layers=-1) == 2
    assert call(out=0x2000) == 2             # out overlaps inputs_embeds
    assert call(ws_bytes=16) == 5
    assert call(layers=None) == 1
    assert call(emb=0x2002) == 2             # inputs_embeds not 16-byte aligned
    assert call(ds=(ctypes.c_void_p * 1)(0x5008)) == 2


def test_step_entry_points_reject_before_launch():
    lib = b.lib()
    assert lib.mhe_rms_norm(None, 0x10, 0x20, 4, 256, 1e-6, None) == 1
    assert lib.mhe_rms_norm(0x10, 0x10, 0x20, 4, 20000, 1e-6, None) == 4
    assert lib.mhe_linear(0x10, 0x20, 0x30, None, 4, 100, 64, None, 0, None) == 4   # n % 32
    assert lib.mhe_linear(0x10, 0x20, 0x30, None, 4, 64, 48, None, 0, None) == 4    # k % 64
    assert lib.mhe_linear(0x1000, 0x900000, 0x1000, None, 4, 64, 64, None, 0, None) == 2  # c aliases a
    assert lib.mhe_linear(0x1000, 0x900000, 0x100000, None, 4, 64, 64, 0x200010, 1 << 20, None) == 5
    assert lib.mhe_linear_swiglu(0x10, None, 0x20, 0x30, 4, 64, 64, None, 0, None) == 1
    assert b.linear_workspace_bytes() >= 256 * 256 * 256 * 4
    assert lib.mhe_attention(0x10, 0x20, 0x30, 0x40, 64, 12, 1, 128, None) == 4  # group 12
    assert lib.mhe_attention(0x10, 0x20, 0x30, 0x40, 0, 8, 1, 128, None) == 2
    assert lib.mhe_deepstack_inject(0x10, 64, 256, 0x20, 65, 0x30, 0x40, 1 << 20, None) == 2
    assert lib.mhe_deepstack_inject(0x10, 64, 256, 0x20, 0, 0x30, 0x40, 1 << 20, None) == 0  # no-op


def test_fp8_entry_points_reject_before_launch():
    lib = b.lib()
    cfg = b.config_from_dims(synth.FULL)
    assert b.workspace_bytes_fp8(cfg, 4096) > b.workspace_bytes(cfg, 4096)
    bad = b.config_from_dims(synth.FULL)
    bad.hidden = 5120 + 64                        # fine for bf16, not a multiple of 128
    assert lib.mhe_workspace_bytes(ctypes.byref(bad), 64) > 0
    assert lib.mhe_workspace_bytes_fp8(ctypes.byref(bad), 64) == 0
    d = 0x100000
    # k % 128 != 0, NULL scale, NULL operand
    assert lib.mhe_linear_fp8(d, d, d, d, d * 8, None, 64, 64, 192, None, 0, None) == 4
    assert lib.mhe_linear_fp8(d, None, d, d, d * 8, None, 64, 64, 256, None, 0, None) == 1
    assert lib.mhe_linear_swiglu_fp8(d, d, None, d, d * 8, 64, 64, 256, None, 0, None) == 1
    parts = (ctypes.c_void_p * 1)(d)
    rows = (ctypes.c_int32 * 1)(16)
    assert lib.mhe_quantize_fp8(parts, rows, 0, 64, d * 8, d * 16, 0x10000, 1 << 20, None) == 2
    assert lib.mhe_quantize_fp8(parts, rows, 1, 60, d * 8, d * 16, 0x10000, 1 << 20, None) == 2
    assert lib.mhe_quantize_fp8(parts, rows, 1, 64, d * 8, None, 0x10000, 1 << 20, None) == 1
    assert lib.mhe_quantize_fp8(parts, rows, 1, 64, d * 8, d * 16, 0x10000, 16, None) == 5
    t = b.MheLayerWeightsFp8(*([0x1000] * 12))
    t.s_down = None
    tiny = b.config_from_dims(synth.TINY)
    rc = lib.mhe_layer_forward_fp8(ctypes.byref(tiny), ctypes.byref(t), 0x2000, 0x3000, 64, 0x10000,
                                   1 << 40, None)
    assert rc == 1 and "s_down" in lib.mhe_last_error().decode()


def test_qnorm_attention_rejects_before_launch():
    lib = b.lib()
    d = 0x100000
    cfg = b.config_from_dims(synth.FULL)
    need = b.qnorm_attention_workspace_bytes(cfg, 64)
    assert need >= 64 * 64 * 8                    # cos/sin of 64 slots per token
    call = lambda c=cfg, **o: lib.mhe_qnorm_attention(
        ctypes.byref(c), o.get("qkv", d), d, d, d, d, d, o.get("seq", 64), o.get("ws", 0x10000),
        o.get("ws_bytes", need), None)
    assert call(qkv=None) == 1
    assert call(qkv=d + 8) == 2                   # not 16-byte aligned
    assert call(seq=0) == 2
    assert call(ws_bytes=need - 1) == 5
    assert call(ws=0x10010) == 5                  # misaligned
    bad = b.config_from_dims(synth.FULL)
    bad.n_heads = 96                              # 12 query heads per kv head
    assert call(bad) == 4


def test_vision_attention_rejects_before_launch():
    import numpy as np
    lib = b.lib()
    d = 0x100000
    grids = np.array([[1, 4, 8], [2, 4, 4]], dtype=np.int32)     # 32 + 32 patches
    g = grids.ctypes.data
    need = b.vision_attention_workspace_bytes(64)
    assert need >= 64 * 32
    call = lambda **o: lib.mhe_vision_attention(
        o.get("q", d), d, d, d * 8, o.get("n", 64), 4, o.get("hd", 72), o.get("g", g),
        o.get("ng", 2), o.get("merge", 2), o.get("ws", 0x10000), o.get("ws_bytes", need), None)
    assert call(q=None) == 1
    assert call(hd=130) == 4                      # head_dim above 128
    assert call(hd=70) == 4                       # not a multiple of 4
    assert call(n=63) == 3                        # grids hold 64 patches
    assert call(g=None) == 1
    assert call(ng=0) == 2
    assert call(merge=0) == 2
    assert call(ws_bytes=need - 1) == 5
    assert call(ws=0x10010) == 5                  # misaligned
    assert b.status_string(3) != b.status_string(2)


def test_deepstack_noalloc_rejects_before_launch():
    lib = b.lib()
    call = lambda **o: lib.mhe_deepstack_inject_noalloc(
        o.get("h", 0x10), o.get("seq", 64), o.get("dim", 256), o.get("mask", 0x20),
        o.get("n_vis", 8), o.get("feat", 0x30), None)
    assert call(seq=(1 << 17) + 1, n_vis=4) == 2          # beyond the static scratch
    assert "static scratch" in lib.mhe_last_error().decode()
    assert call(seq=0) == 2
    assert call(dim=100) == 2
    assert call(n_vis=65) == 2
    assert call(h=None) == 1
    assert call(mask=None) == 1
    assert call(n_vis=0) == 0                             # no-op, nothing launched
