"""Plain CPU oracle for the offloaded-expert MoE step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import anything from here.  The product
path (the HIP library and its Python binding) never imports, links or calls
this package, and this package imports nothing from the product.

Every function is a slow, direct restatement of what the source pages say the
step computes, in float64 where floating point is involved:

  * ``formulas``  - the benchmark arithmetic (miss count, copy MiB, GB/s, tok_ms)
  * ``lru``       - ensure_experts: the global LRU slot remap over flat ids
  * ``copy``      - copy_missing: per-bank row gather for each miss
  * ``decode``    - bit-field decoders for bf16 / e4m3 / e8m0 / e2m1 / fp16
  * ``schema``    - the per-format bank list and row sizes
  * ``ffn``       - the SwiGLU expert FFN with top-k weighted combine
  * ``route``     - softmax top-k routing, renormalised
  * ``checksum``  - position-weighted sampled checksum of a bank
  * ``prefill``   - the whole-layer streamed buffer and its FFN

Page names used in citations:
  "FreeToken architecture walk-through"  - the architecture page (HTTP API to
      CUDA kernels), sections numbered 1-8 as on the page.
  "FreeToken MoE benchmark guide"        - the offline benchmark guide,
      sections 1-6 with the page's own sub-numbers (e.g. 4.3).

Parity status: every function here has at least one pin in
``tests/test_oracle_*.py`` except the readings listed as "parity unpinned" in
the module that makes them (LRU tie-breaks, nibble order, transposed MXFP4
layout, routing at near-ties).
"""
from . import formulas, schema, decode, lru, copy, route, ffn, checksum, prefill  # noqa: F401
