"""Plain, slow CPU oracle for one block-diffusion denoising step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything under ``oracle/``; only the tests, the smoke check and the
benchmark's CPU-baseline leg do.  The oracle shares no code with the GPU path:
it receives plain numpy arrays (the same bytes the GPU consumes, decoded to
fp64) and computes every step by its textbook definition in fp64.

What it follows, by source page:

* "DiffusionGemma Technical Report" (write-up of the paper), Figure 4: the
  three-stage pipeline -- the prompt is encoded causally into a KV cache; a
  noisy 256-token canvas is refined by a decoder that attends bidirectionally
  inside the canvas and to the cached context; the finished canvas is encoded
  causally again and appended to the cache.
* Same page, "What they did": the canvas starts as random noise and the whole
  block is refined in parallel; an entropy-bounded sampler with adaptive
  stopping ends denoising once predictions are confident.
* Same page, Table 1: mixture-of-experts transformer, 8 of 128 experts active,
  262k-token vocabulary.
* "diffusiongemma" model card, "Model Overview" and feature list: causal
  encoder for the prompt, bidirectional decoder over the canvas with
  cross-attention to the cache, block-autoregressive generation, the
  "Entropy Bound" sampler.

The pages give no layer-level formulas; the readings taken where they are
silent are listed in ``oracle/model.py``'s module docstring.

Parity status per function: every public function of ``oracle.model`` is
pinned by the not-gpu tests under ``tests/`` against closed forms, invariants,
brute force on tiny inputs or hand-worked fixtures in ``tests/golden/``.
"""
from .model import (  # noqa: F401
    CANVAS,
    Shapes,
    rmsnorm,
    canvas_attention,
    router_topk,
    moe_mixture,
    moe_layer,
    lm_head_stats,
    lm_logits,
    linear_w8a8,
    projection,
    lm_head_sample,
    gumbel,
    temperature,
    eb_select,
    denoise_step,
    commit_block,
    accumulate_in,
    ar_step,
    expert_matrix,
)
from .numerics import (round_bf16, decode_e4m3, encode_e4m3,  # noqa: F401
                       quantize_rows_e4m3, kv_cache_values)
