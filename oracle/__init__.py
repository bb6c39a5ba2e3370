"""CPU fp64 oracle for the dropless routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never calls it, and
it shares no code with the GPU library: it has its own routing, its own
MXFP8 codecs and its own planner simulation, written from the pages' math.

Modules
  moe      routing metadata, expert SwiGLU FFN, combine, backward (bf16/fp32
           inputs are decoded exactly and all arithmetic is fp64)
  mx       MXFP8 codecs (E4M3 "FN" values, E8M0 block scales) and the
           quantization-faithful MXFP8 forward/backward
  planner  saved-state byte accounting and the save/replay decision

Parity status
  pinned   routing, expert math, combine, backward, E4M3 decoding and rounding,
           planner inequality, FLOP count (see tests/test_oracle_*.py)
  parity unpinned
           the E8M0 scale-selection rule (the pages say the producer picks the
           scale but not how; the rule here is a documented choice, checked
           only for its stated property), the GPU's bf16 rounding points
           (bounded by tolerance only) and fp32 summation order.
"""
