"""CPU oracle for the routed-expert NVFP4 (W4A4) MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg may use
it.  It shares no code with the HIP library (no kernels, headers, tables or
helpers); the two meet only through the seeded generators in ``synth``.

What it computes (the engine on the pages: the release post "capy-flash
v0.7.1: a 125B MoE on 64 GB of RAM ...", sections "What shipped" and "Why it
matters"; the blog "Capy Flash ... two consumer GPUs", section "Where the
experts live"; the forum repost, paragraph "Where it stands"):

  router   logits = x . W_r^T (+ bias), softmax over all experts, keep top-k,
           renormalise                                     -> oracle.router
  W4A4     x and every expert weight block-quantized to NVFP4 (E2M1 codes,
           an E4M3 scale per 16 elements, an FP32 tensor scale) -> oracle.nvfp4
  FFN      per picked expert: SwiGLU gate/up, SiLU gate, re-quantized h,
           down projection                                  -> oracle.ffn
  combine  y = residual + sum_i w_i o_i, rounded once to bf16 -> oracle.ffn
  permute  stable token-by-expert counting sort              -> oracle.permute
  codebook 3-bit group-128 fp16-codebook gate/up weights     -> oracle.codebook

Arithmetic: quantizers follow fp32 IEEE round-to-nearest-even exactly as the
steps are written (no fused multiply-add); matmuls run in fp64 on exactly
dequantized values, so results are the exact quantized computation up to fp64
rounding order.  Every function is pinned by tests under ``tests/`` that do
not reuse its code (tables, library routines, brute force in exact rational
arithmetic, closed forms and invariants).
"""
from . import formats, nvfp4, router, permute, ffn, codebook  # noqa: F401
