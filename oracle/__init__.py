"""CPU oracle for the NVFP4 W4A4 MoE expert GEMM with Residual Activation
Compensation (QUADS, arXiv 2607.15810).

TEST INFRASTRUCTURE ONLY.  This is a plain, slow, float64 numpy statement of
what the HIP library computes.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the library under
fp4_quantized_gemm_amd/ never does, and shares no code with it.

Modules:
  formats  E2M1, E4M3 and bfloat16 encode/decode from their bit definitions
  nvfp4    tensor/block scales, quantize, dequantize, residual, channel
           scores, channel selection, weight QDQ, nibble packing
  moe      router top-k + softmax, expert-major permutation, SwiGLU, combine
  gemm     expert-grouped W4A4 GEMM plus the residual correction, and the
           trainer-side W4A16 product with the same dequantized weights
  layer    the whole MoE layer chained from the pieces above
  fp8      the FP8 (E4M3) W8A8 baseline: per-tensor quantization and the
           expert-grouped product

Every function is pinned by tests under tests/ against facts that do not come
from the oracle itself (bit definitions, exact rational arithmetic, library
routines, closed forms and invariants).
"""
from . import formats, fp8, gemm, layer, moe, nvfp4  # noqa: F401
