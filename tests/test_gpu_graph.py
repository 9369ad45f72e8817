"""mhe_encode under HIP graph capture.

The library allocates nothing and issues only kernels and one device-to-device
copy on the caller's stream, so a whole encode can be captured once and
replayed. The captured four-layer seq-2048 image stack (320-wide GEMM tiles,
DeepStack levels) must give, on every replay, bit-for-bit the eager encode's
output — with unrelated eager work and host synchronisations between the
replays — and must read its inputs afresh on each replay.
"""

import pytest
import torch

from multimodal_encoder_prefill_amd import binding as b
from multimodal_encoder_prefill_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_encode_graph_replays_match_eager():
    wl = synth.WORKLOADS["image_s2048_l4"]
    print(f"graph capture of mhe_encode, workload {wl.key}", flush=True)
    layers = [synth.layer_weights(wl, l, DEV) for l in range(wl.n_layers)]
    emb = synth.embeddings(wl, DEV)
    pos = torch.from_numpy(synth.positions(wl)).to(DEV)
    mask = torch.from_numpy(synth.visual_mask(wl)).to(DEV)
    ds = [synth.deepstack_features(wl, i, DEV) for i in range(wl.n_ds)]
    cfg = b.config_from_dims(wl.dims)
    nbytes = b.workspace_bytes(cfg, wl.seq)
    ws = torch.empty(nbytes, device=DEV, dtype=torch.uint8)
    tables = [b.layer_table(w) for w in layers]

    def run(out):
        b.encode(cfg, tables, emb, pos, wl.seq, out, ws, nbytes, visual_mask=mask, n_vis=wl.n_vis,
                 deepstack=ds)

    eager = torch.empty_like(emb)
    run(eager)
    torch.cuda.synchronize()

    out = torch.empty_like(emb)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out)
    torch.cuda.synchronize()

    scratch = torch.randn(4096, 4096, device=DEV)
    for i in range(3):
        out.fill_(float("nan"))
        scratch = scratch @ scratch.T * 1e-3          # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        print(f"replay {i}: bit-identical to eager = {torch.equal(out, eager)}", flush=True)
        assert torch.equal(out, eager)

    # new inputs in the captured buffers: the replay computes on them
    emb.mul_(-0.5)
    eager2 = torch.empty_like(emb)
    run(eager2)
    g.replay()
    torch.cuda.synchronize()
    assert not torch.equal(eager2, eager)
    assert torch.equal(out, eager2)
