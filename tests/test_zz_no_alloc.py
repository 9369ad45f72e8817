"""The allocation-free DeepStack entry point against the workspace one.

mhe_deepstack_inject_noalloc runs the same two kernels as mhe_deepstack_inject
with the visual index list in the library's static device scratch instead of
a caller workspace, so its output must be bit-identical to the workspace
form's (and within the DeepStack bar of the oracle). Two calls in a row, the
second on a smaller input, show that the scratch left by the first call does
not leak into the second.
"""

import numpy as np
import pytest
import torch

import oracle
from helpers import f64, report

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(seq, dim, density, seed):
    from multimodal_encoder_prefill_amd import binding as b
    rng = np.random.default_rng(seed)
    mask = (rng.random(seq) < density).astype(np.uint8)
    n_vis = int(mask.sum())
    g = torch.Generator(device=DEV).manual_seed(seed)
    h = torch.randn(seq, dim, generator=g, device=DEV).to(torch.bfloat16)
    feat = torch.randn(max(n_vis, 1), dim, generator=g, device=DEV).to(torch.bfloat16)
    m = torch.from_numpy(mask).to(DEV)
    h_ws = h.clone()
    ws = torch.empty(seq * 4 + 512, device=DEV, dtype=torch.uint8)
    b.deepstack_inject(h_ws, seq, dim, m, n_vis, feat, ws, ws.numel())
    h_na = h.clone()
    b.deepstack_inject_noalloc(h_na, seq, dim, m, n_vis, feat)
    torch.cuda.synchronize()
    return h, h_ws, h_na, mask, feat, n_vis


def test_noalloc_matches_workspace_form_twice_shrinking():
    print("deepstack noalloc: seq 4096 dim 5120, then seq 333 dim 256", flush=True)
    for seq, dim, density, seed in [(4096, 5120, 0.5, 1), (333, 256, 0.2, 2)]:
        h, h_ws, h_na, mask, feat, n_vis = _case(seq, dim, density, seed)
        assert torch.equal(h_na, h_ws), (seq, dim)
        ref = oracle.deepstack_add(f64(h), mask, f64(feat)[:n_vis])
        assert report(f"deepstack noalloc seq {seq}", f64(h_na), ref)[0] <= 4e-3
        assert np.array_equal(f64(h_na)[mask == 0], f64(h)[mask == 0])


def test_noalloc_short_mask_after_long_call():
    """A call whose mask holds fewer visual tokens than n_vis right after a
    call that filled the scratch with valid indices: the extra feature rows
    must still be ignored (the index kernel rewrites every entry it reads)."""
    from multimodal_encoder_prefill_amd import binding as b
    _case(2048, 512, 0.9, 3)                      # fills ~1840 scratch entries
    seq, dim = 128, 256
    mask = np.zeros(seq, np.uint8); mask[10:20] = 1
    g = torch.Generator(device=DEV).manual_seed(4)
    h0 = torch.randn(seq, dim, generator=g, device=DEV).to(torch.bfloat16)
    feat = torch.randn(16, dim, generator=g, device=DEV).to(torch.bfloat16)
    m = torch.from_numpy(mask).to(DEV)
    h = h0.clone()
    b.deepstack_inject_noalloc(h, seq, dim, m, 16, feat)
    torch.cuda.synchronize()
    ref = f64(h0); ref[10:20] += f64(feat)[:10]
    assert report("noalloc short mask", f64(h), ref)[0] <= 4e-3
    assert np.array_equal(f64(h)[20:], f64(h0)[20:]) and np.array_equal(f64(h)[:10], f64(h0)[:10])
