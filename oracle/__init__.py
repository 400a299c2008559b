"""CPU oracle for the fused grouped W4A16 mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
implementation of what the layer computes, written in numpy with float64
arithmetic.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import it; the product path (the HIP library and its Python binding)
never does, and it shares no code with it.

What is computed, following ExactMoE (page "Every Expert Counts: ExactMoE for
Memory-Efficient W4A16 Inference", Abstract): routed-expert weights are held as
symmetric four-bit integers with one scale per 128 input channels, the router
stays in BF16 and its top-k procedure is unchanged, and every selected expert
is executed (none pruned or substituted).  The pages leave the quantiser's
scale rule, the packed layout, the activation, the top-k tie rule, the
normalisation of routing weights, the combine and the slot-cache policy open;
each module states the reading it takes.

Modules
  bf16       bf16 bit decoding and round-to-nearest-even encoding
  quant      group-128 symmetric int4 quantise / dequantise, packed layout v1
  route      router logits, top-k selection, routing weights
  align      expert-sorted permutation (stable counting sort)
  ffn        per-pair SwiGLU expert FFN, routing-weighted combine, whole layer
  slot_cache LRU simulator for the GPU-resident expert slot cache

Pinning status: every function here is pinned by a CPU test against brute
force, closed forms, invariants or an independent formulation (tests/test_oracle_*.py).
The pages print no worked example and no intermediate value, so no function is
pinned to numbers from the pages themselves.
"""
from . import bf16, quant, route, align, ffn, slot_cache  # noqa: F401
