"""CPU oracle for the block-quantized routed-MoE path.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
reference: it decodes every block format to its exact real value in float64,
and runs the MoE projection with float64 accumulation. Only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use it.
It shares no code with the GPU library (``bit_quantized_moe_dequant_amd``) and
imports nothing from it; inputs come from the caller.

Modules:
  codecs   element codecs (e2m1, e4m3fn, e8m0, fp16, bf16) from their definitions
  formats  per-format decode of whole tensors (source layouts) and sizes: MXFP4,
           NVFP4, Q2_K, IQ2_XXS, FP8 block-128, FP8 block-32, MXFP8
  convert  the lossless MXFP4 -> NVFP4 re-encode and its exact inverse
  mxfp8    MXFP8 activation quantisation (E4M3 elements, e8m0 per 32)
  moe      routed-MoE layer, dense FP8 linear, and the W4A8 prefill chain

Parity unpinned (nothing in this environment can check them; see the design
notes): ggml fidelity of the Q2_K crumb order and of the IQ2_XXS bit layout,
scale offset, scale factor, sign rule and codebook values. Every function below is
pinned by the CPU tests against closed forms, library decoders, brute force or
worked examples; the IQ2_XXS and Q2_K decoders are pinned only against the layout
as read here, not against ggml.
"""
from . import codecs, formats, convert, mxfp8, moe  # noqa: F401
