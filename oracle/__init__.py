"""CPU oracle for the Qwen3-VL layer-50 text-decoder prefill.

TEST INFRASTRUCTURE ONLY. This package is the slow, obviously correct
reference that the HIP path is checked against. Only the test-suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path (``multimodal_encoder_prefill_amd``) never imports,
calls or links anything here, and nothing here imports the product path.

Everything is float64 NumPy. Inputs are taken as given (the callers pass
bf16-representable values); no step rounds to bf16. Each function names the
page and the class/function on it whose computation it follows:

* "H3 encoder page" = the vllm-omni source page
  ``vllm_omni/diffusion/models/minimax_h3/encoder.py`` (MiniMax H3 Qwen3-VL
  layer-50 text/vision encoder);
* "vLLM Qwen3-VL page" = ``vllm/model_executor/models/qwen3_vl.py``;
* "SGLang Qwen3-VL page" = ``python/sglang/srt/models/qwen3_vl.py``.

``oracle.vision`` holds the page's Qwen3-VL vision tower (patch embedding,
interpolated position embeddings, 2-D rotary, non-causal per-frame attention
blocks, the merger and the DeepStack mergers).

``oracle.fp8`` holds the online-FP8 reading of the decoder's linears
(per-tensor E4M3 quantisation of weights and activations).

``oracle.frontend`` holds the token-level front end of the same page
(token types, embedding gather with visual placeholder scatter, the joint
DeepStack order and the multimodal rotary position ids).

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, invariants, hand-derived fixtures under
``tests/golden/`` and independent library routines (torch's ``rms_norm`` and
``scaled_dot_product_attention``). The full 50-layer values on synthetic
weights are pinned only through the composition of those parts (the pages
print no output values).
"""

from .qwen3vl_text import (  # noqa: F401
    ModelDims,
    LayerWeights,
    rms_norm,
    mrope_slot_axes,
    rope_inv_freq,
    rope_cos_sin,
    apply_rope,
    silu,
    causal_gqa_attention,
    decoder_layer,
    deepstack_add,
    encode,
    layer_param_count,
)
from .positions import text_and_grid_positions  # noqa: F401
from . import frontend  # noqa: F401
from . import vision  # noqa: F401
from . import fp8  # noqa: F401
