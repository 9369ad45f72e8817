"""Seeded synthetic inputs for the Qwen3-VL layer-50 text-decoder prefill.

This module only draws numbers and lays out index data: it holds none of the
decoder's arithmetic, and both the HIP path's callers and the CPU oracle's
tests take their inputs from it.

No trained checkpoint, tokenizer, image or video is available, so seeded
random tensors with the model's shapes stand in for them:

* linear weights ~ N(0, 0.02), RMSNorm gains ~ U(0.5, 1.5), input embeddings
  and DeepStack features ~ N(0, 1); all drawn in float32 and rounded to bf16
  (round-to-nearest-even), the storage type of the path;
* the visual tokens form one contiguous block in the middle of the sequence;
* positions follow the multimodal rotary rule of the H3 encoder page
  (``_get_rope_index``): text runs count up on all three axes, a visual block
  with merged grid (t, h, w) starting at position s gives the token at frame
  f, row r, column c the ids (s+f, s+r, s+c), and the following text resumes
  at s + max(h, w).

Each tensor has its own generator seeded from (workload, layer, tensor id),
so a single layer can be regenerated without drawing the rest of the stack.
Draws use torch's generator for the requested device; values are
deterministic per device type (a CPU draw and a GPU draw of the same tensor
differ), so callers that compare two implementations draw once and copy.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np
import torch

_BASE_SEED = 20261202

# tensor ids inside a layer
TENSOR_IDS = {
    "w_q": 0, "w_k": 1, "w_v": 2, "w_o": 3, "w_gate": 4, "w_up": 5, "w_down": 6,
    "ln_in": 7, "ln_post": 8, "q_norm": 9, "k_norm": 10,
}
_EMBED_ID = 100
_DEEPSTACK_ID = 200


@dataclass(frozen=True)
class Dims:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    rms_eps: float = 1e-6
    rope_theta: float = 5e6
    mrope_section: Tuple[int, int, int] = (24, 20, 20)

    @property
    def q_width(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim


@dataclass(frozen=True)
class Workload:
    key: str
    index: int
    dims: Dims
    seq: int
    n_layers: int
    # ("text", n) or ("visual", (t, h, w)) with the merged grid
    segments: Tuple = field(default_factory=tuple)
    n_ds: int = 0
    description: str = ""

    @property
    def n_vis(self) -> int:
        return sum(int(np.prod(s)) for k, s in self.segments if k == "visual")


FULL = Dims(hidden=5120, n_heads=64, n_kv_heads=8, head_dim=128, intermediate=25600,
            rms_eps=1e-6, rope_theta=5e6)
TINY = Dims(hidden=256, n_heads=4, n_kv_heads=1, head_dim=64, intermediate=1024,
            rms_eps=1e-6, rope_theta=1e6)

WORKLOADS: Dict[str, Workload] = {
    w.key: w for w in [
        Workload("tiny", 0, TINY, 64, 2, (("text", 64),), 0,
                 "tiny 2-layer decoder, seq 64 text-only"),
        Workload("layer1_s512", 1, FULL, 512, 1, (("text", 512),), 0,
                 "one full-width layer, seq 512 text-only"),
        Workload("image_s2048_l4", 2, FULL, 2048, 4,
                 (("text", 512), ("visual", (1, 32, 32)), ("text", 512)), 3,
                 "4 full-width layers, seq 2048 with a 1x32x32 image block, 3 DeepStack levels"),
        Workload("image_s4096_l50", 3, FULL, 4096, 50,
                 (("text", 1024), ("visual", (1, 32, 64)), ("text", 1024)), 3,
                 "50 full-width layers, seq 4096 with a 1x32x64 image block, 3 DeepStack levels"),
        Workload("video_s16384_l50", 4, FULL, 16384, 50,
                 (("text", 1024), ("visual", (14, 32, 32)), ("text", 1024)), 3,
                 "50 full-width layers, seq 16384 with a 14x32x32 video block, 3 DeepStack levels"),
    ]
}


def custom_workload(dims: Dims, seq: int, n_layers: int, segments=None, n_ds: int = 0,
                    key: str = "custom", index: int = 99) -> Workload:
    """A workload of arbitrary shape (used by tests for ragged sizes)."""
    if segments is None:
        segments = (("text", seq),)
    wl = Workload(key, index, dims, seq, n_layers, tuple(segments), n_ds, key)
    total = sum(int(np.prod(s)) if k == "visual" else int(s) for k, s in wl.segments)
    if total != seq:
        raise ValueError(f"segments cover {total} tokens, seq is {seq}")
    return wl


def _seed(wl: Workload, layer: int, tid: int) -> int:
    return ((_BASE_SEED * 1000 + wl.index) * 1000 + (layer + 1)) * 1000 + tid


def _gen(wl: Workload, layer: int, tid: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(_seed(wl, layer, tid))
    return g


def _normal(shape, std, wl, layer, tid, device) -> torch.Tensor:
    g = _gen(wl, layer, tid, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def _uniform(shape, lo, hi, wl, layer, tid, device) -> torch.Tensor:
    g = _gen(wl, layer, tid, device)
    x = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(hi - lo).add_(lo)
    return x.to(torch.bfloat16)


def layer_shapes(d: Dims) -> Dict[str, Tuple[int, ...]]:
    return {
        "ln_in": (d.hidden,),
        "w_q": (d.q_width, d.hidden),
        "w_k": (d.kv_width, d.hidden),
        "w_v": (d.kv_width, d.hidden),
        "q_norm": (d.head_dim,),
        "k_norm": (d.head_dim,),
        "w_o": (d.hidden, d.q_width),
        "ln_post": (d.hidden,),
        "w_gate": (d.intermediate, d.hidden),
        "w_up": (d.intermediate, d.hidden),
        "w_down": (d.hidden, d.intermediate),
    }


def layer_weights(wl: Workload, layer: int, device="cpu") -> Dict[str, torch.Tensor]:
    """bf16 weights of one decoder layer (linear N(0,0.02), gains U(0.5,1.5))."""
    out = {}
    for name, shape in layer_shapes(wl.dims).items():
        tid = TENSOR_IDS[name]
        if name.startswith("w_"):
            out[name] = _normal(shape, 0.02, wl, layer, tid, device)
        else:
            out[name] = _uniform(shape, 0.5, 1.5, wl, layer, tid, device)
    return out


def embeddings(wl: Workload, device="cpu") -> torch.Tensor:
    """Input embeddings [S, H] bf16 ~ N(0, 1)."""
    return _normal((wl.seq, wl.dims.hidden), 1.0, wl, -1, _EMBED_ID, device)


def deepstack_features(wl: Workload, level: int, device="cpu") -> torch.Tensor:
    """DeepStack level features [n_vis, H] bf16 ~ N(0, 1)."""
    return _normal((wl.n_vis, wl.dims.hidden), 1.0, wl, -1, _DEEPSTACK_ID + level, device)


def visual_mask(wl: Workload) -> np.ndarray:
    """uint8 [S]: 1 on visual tokens."""
    parts: List[np.ndarray] = []
    for kind, spec in wl.segments:
        n = int(np.prod(spec)) if kind == "visual" else int(spec)
        parts.append(np.full(n, 1 if kind == "visual" else 0, dtype=np.uint8))
    return np.concatenate(parts) if parts else np.zeros(0, np.uint8)


def positions(wl: Workload) -> np.ndarray:
    """int32 [3, S] (T, H, W) position ids of the workload's segments."""
    cols = []
    cur = 0
    for kind, spec in wl.segments:
        if kind == "text":
            n = int(spec)
            ramp = cur + np.arange(n, dtype=np.int64)
            cols.append(np.stack([ramp, ramp, ramp]))
            cur += n
        else:
            t, h, w = (int(x) for x in spec)
            f, r, c = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")
            cols.append(np.stack([cur + f.ravel(), cur + r.ravel(), cur + c.ravel()]))
            cur += max(h, w)
    return np.concatenate(cols, axis=1).astype(np.int32)


def random_positions(seq: int, max_pos: int, seed: int) -> np.ndarray:
    """int32 [3, S] with independent axes (exercises every rotary slot rule)."""
    rng = np.random.default_rng([_BASE_SEED, seed])
    return rng.integers(0, max_pos, size=(3, seq)).astype(np.int32)


# ---- token-level inputs (ids, embedding table, vision-tower outputs) ----

_TABLE_ID = 300
_FEATURE_ID = 400


def prompt_ids(runs, image_token_id: int, video_token_id: int, text_vocab: int,
               seed: int) -> np.ndarray:
    """int32 token ids for runs ("text" | "image" | "video", token count), in order.

    Text ids are drawn uniformly from [0, text_vocab) (callers keep the
    placeholder ids outside that range); image / video runs are the
    placeholder ids."""
    rng = np.random.default_rng([_BASE_SEED, _TABLE_ID, seed])
    parts = []
    for kind, n in runs:
        if kind == "text":
            parts.append(rng.integers(0, text_vocab, size=int(n)))
        else:
            tok = image_token_id if kind == "image" else video_token_id
            parts.append(np.full(int(n), tok))
    return np.concatenate(parts).astype(np.int32)


def token_table(vocab: int, hidden: int, seed: int, device="cpu") -> torch.Tensor:
    """Embedding table [vocab, hidden] bf16 ~ N(0, 1)."""
    g = torch.Generator(device=device)
    g.manual_seed(_BASE_SEED * 1000 + _TABLE_ID + seed)
    return torch.randn(vocab, hidden, generator=g, device=device).to(torch.bfloat16)


def feature_rows(n: int, hidden: int, seed: int, device="cpu") -> torch.Tensor:
    """Vision-tower output rows [n, hidden] bf16 ~ N(0, 1)."""
    g = torch.Generator(device=device)
    g.manual_seed(_BASE_SEED * 1000 + _FEATURE_ID + seed)
    return torch.randn(n, hidden, generator=g, device=device).to(torch.bfloat16)


_FP8_ID = 600


def fp8_codes(shape, seed: int, device="cpu", exp_lo: int = 3, exp_hi: int = 12) -> torch.Tensor:
    """Random E4M3 byte codes (uint8): random sign and mantissa, exponent field
    uniform in [exp_lo, exp_hi] (magnitudes 2^(exp_lo-7) .. 2^(exp_hi-6)), so
    the NaN codes never occur."""
    g = torch.Generator(device=device)
    g.manual_seed(_BASE_SEED * 1000 + _FP8_ID + seed)
    sign = torch.randint(0, 2, shape, generator=g, device=device, dtype=torch.int32)
    exp = torch.randint(exp_lo, exp_hi + 1, shape, generator=g, device=device, dtype=torch.int32)
    man = torch.randint(0, 8, shape, generator=g, device=device, dtype=torch.int32)
    return ((sign << 7) | (exp << 3) | man).to(torch.uint8)


# ---- vision tower inputs (patch pixels and random-init tower weights) ----

_VISION_ID = 500


@dataclass(frozen=True)
class VisionDims:
    """Vision tower sizes; `intermediate` is the stored (zero-padded) MLP width,
    `mlp_width` the model's."""
    hidden: int
    n_heads: int
    mlp_width: int
    intermediate: int
    depth: int
    patch: int
    temporal_patch: int
    in_channels: int
    merge: int
    out_hidden: int
    pos_side: int
    deepstack: Tuple[int, ...]

    @property
    def patch_dim(self) -> int:
        return self.in_channels * self.temporal_patch * self.patch * self.patch

    @property
    def merged_hidden(self) -> int:
        return self.hidden * self.merge * self.merge


# Qwen3-VL vision config (not printed on the pages): 27 blocks of width 1152,
# 16 heads of 72, MLP 4304 (stored as 4352), 16x16x2 patches of 3 channels,
# merge 2, 48x48 position table, DeepStack after blocks 8, 16, 24.
VISION_FULL = VisionDims(hidden=1152, n_heads=16, mlp_width=4304, intermediate=4352, depth=27,
                         patch=16, temporal_patch=2, in_channels=3, merge=2, out_hidden=5120,
                         pos_side=48, deepstack=(8, 16, 24))
# small tower with the same head_dim (72) and a padded MLP width
VISION_TINY = VisionDims(hidden=576, n_heads=8, mlp_width=1000, intermediate=1024, depth=3,
                         patch=8, temporal_patch=2, in_channels=3, merge=2, out_hidden=256,
                         pos_side=8, deepstack=(0, 2))


def _vgen(seed: int, tid: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_BASE_SEED * 1000 + _VISION_ID + seed * 100 + tid)
    return g


def vision_weights(vd: VisionDims, seed: int = 0, device="cpu") -> Dict:
    """Random-init tower: linear weights and biases N(0, 0.02), norm weights
    U(0.5, 1.5), norm biases N(0, 0.1), position table N(0, 0.5); the MLP is
    drawn at its model width and stored zero-padded to `intermediate`."""
    tid = [0]

    def nrm(shape, std):
        tid[0] += 1
        g = _vgen(seed, tid[0], device)
        return (torch.randn(*shape, generator=g, device=device) * std).to(torch.bfloat16)

    def uni(n):
        tid[0] += 1
        g = _vgen(seed, tid[0], device)
        return (0.5 + torch.rand(n, generator=g, device=device)).to(torch.bfloat16)

    H, I, Ipad, M = vd.hidden, vd.mlp_width, vd.intermediate, vd.merged_hidden

    def padded(t, rows=None, cols=None):
        out = torch.zeros(rows if rows is not None else t.shape[0],
                          *(([cols] if cols is not None else list(t.shape[1:]))),
                          dtype=t.dtype, device=t.device)
        if t.dim() == 1:
            out[:t.shape[0]] = t
        elif cols is not None:
            out[:, :t.shape[1]] = t
        else:
            out[:t.shape[0]] = t
        return out

    def merger(post):
        nd = M if post else H
        return {"norm_w": uni(nd), "norm_b": nrm((nd,), 0.1), "fc1_w": nrm((M, M), 0.02),
                "fc1_b": nrm((M,), 0.02), "fc2_w": nrm((vd.out_hidden, M), 0.02),
                "fc2_b": nrm((vd.out_hidden,), 0.02)}

    w = {"patch_w": nrm((H, vd.patch_dim), 0.02), "patch_b": nrm((H,), 0.02),
         "pos_table": nrm((vd.pos_side * vd.pos_side, H), 0.5), "blocks": []}
    for _ in range(vd.depth):
        fc1_w, fc1_b, fc2_w = nrm((I, H), 0.02), nrm((I,), 0.02), nrm((H, I), 0.02)
        w["blocks"].append({
            "norm1_w": uni(H), "norm1_b": nrm((H,), 0.1), "qkv_w": nrm((3 * H, H), 0.02),
            "qkv_b": nrm((3 * H,), 0.02), "proj_w": nrm((H, H), 0.02), "proj_b": nrm((H,), 0.02),
            "norm2_w": uni(H), "norm2_b": nrm((H,), 0.1),
            "fc1_w": padded(fc1_w, rows=Ipad), "fc1_b": padded(fc1_b, rows=Ipad),
            "fc2_w": padded(fc2_w, cols=Ipad), "fc2_b": nrm((H,), 0.02)})
    w["merger"] = merger(False)
    w["deepstack"] = [merger(True) for _ in vd.deepstack]
    return w


def vision_pixels(n: int, vd: VisionDims, seed: int = 0, device="cpu") -> torch.Tensor:
    """Patch pixels [n, patch_dim] bf16 ~ N(0, 1) (normalised image values)."""
    g = _vgen(seed, 99, device)
    return torch.randn(n, vd.patch_dim, generator=g, device=device).to(torch.bfloat16)
