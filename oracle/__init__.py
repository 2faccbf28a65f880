"""Plain, slow CPU oracle of block-verify speculative decoding.

TEST INFRASTRUCTURE ONLY.  This package is the reference the HIP path is
checked against; it shares no code with the HIP path and imports nothing from
it.  Only the test suite, the smoke entry point and the benchmark's CPU
baseline may import it.  No product path may call into it.

Arithmetic is float64 throughout (bf16 weights are upcast exactly), numpy
only, no blocking or fusion beyond the definitions.

Modules
  model   decoder forward, KV cache, chunked prefill
  accept  greedy longest-prefix and modified rejection sampling
  philox  Philox4x64-10 counter-based generator and its uniforms
  q4      dequantisation of the 4-bit group-64 substitute weights
  spec    speculative rounds (verify + accept + trim + repair) and AR decode
"""
