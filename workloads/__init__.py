"""Seeded synthetic workloads for speculative-draft branch attention.

This package only builds *inputs*: the packed-batch structure (sequence
offsets, query positions, branch anchors, branch row offsets, branch modes)
and seeded random tensors rounded to bf16.  It holds none of the attention
arithmetic, so both the CPU oracle (``oracle/``) and the HIP library can be
fed from it without sharing any code path.

The shapes follow the workloads the pages measure the operator on: EAGLE-3
training-time-test (TTT) branches of depth k anchored at every token, and
DFlash-style draft blocks anchored every 16th token, over variable-length
packed batches up to 256K tokens (evolve.pub review, "Key claims under review"
and "Strengths"; rcap.io explainer, results paragraph on the CP kernel).
"""
from .configs import Workload, get, names, TTT, BLOCK  # noqa: F401
from .inputs import make_inputs, bf16_round_bits, bf16_bits_to_f32  # noqa: F401
