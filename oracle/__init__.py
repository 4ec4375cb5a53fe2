"""Oracle for the routed MoE FFN layer with group-quantised experts.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, CPU implementation of
what the layer computes, written to be checked by eye against the pages. Only
the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it; the product path (the HIP library and its Python binding) never
does, and this package never imports the product.

Arithmetic is fp64 except where the method itself fixes fp32 steps (the
quantisers, whose integer codes are decided in fp32 so that a GPU can reach the
same codes bit for bit).

Sources (the pages; cited by title and section):
  * "I ran a 7B Mixture-of-Experts LLM in a language I built" (dev.to), sections
    "Mixture-of-Experts" (top-8 of 64 experts) and "It works - and it's exact"
    (an fp32 numpy reference used as the oracle of an int8 engine).
  * "mtlm-7m-base" (huggingface.co), sections "Files" (int8 export with group
    size 32; max abs quantisation error 1.7e-3) and "What is and is not machin"
    (SwiGLU, SiLU; a float64 numpy oracle).
  * "Show HN: Getting GLM-5.2 running on my slow computer" (note.crab.center), section
    "What's implemented": a sigmoid router of the DeepSeek-V3 kind
    (noaux_tc selection, a routed scaling factor), a shared expert, integer
    dots on int8 activations quantised the Q8_0 way, int8 and packed int4
    weights dequantised on use, one read of each selected expert per batch
    in prefill and verification.

Modules:
  quant     group-32 weight quantiser, int4 packing, Q8_0 activations
  router    softmax top-k and sigmoid noaux_tc routers
  dispatch  per-expert counts and the stable token permutation
  ffn       SwiGLU expert FFN in fp32-activation and Q8_0 modes
  layer     the whole layer: route, dispatch, experts, combine
"""
from . import quant, router, dispatch, ffn, layer  # noqa: F401
