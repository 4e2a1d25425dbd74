"""CPU oracle for the Pulsar Attention hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy definitions of what the hot path
computes, written from "Dropping the Anchor: Statistical Context
Summarization for Distributed Systems via Pulsar Attention" (Section 2
Method, Figure 2, Section 2.2 Query phase) and the review of Star Attention
(arXiv 2411.17116; its summary of the anchor and of the distributed
online-softmax aggregation).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import anything from this package.  The GPU library never calls it, shares no
code with it, and this package imports nothing from the GPU library.

Floating point is float64 throughout.  Two roundings to bfloat16 are part of
the definitions, because the method runs a bf16 model: the inputs are bf16
values, and the rotated queries and keys (the attention operands) are bf16.

Modules:
  bf16       -- round-to-nearest-even to bfloat16, from float64
  selection  -- document frequency, Max-IDF chunk scores, top-k, prefix lists
  rope       -- rotary position embedding with float64 angles
  attention  -- Phase-1 encoding, Phase-2 per-shard partials, exact LSE merge
"""
