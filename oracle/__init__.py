"""CPU oracle: a plain, slow, fp64 definition of the batch-invariant logprob
recompute forward.

THIS IS TEST INFRASTRUCTURE.  Only the tests, the package's smoke entry and
the CPU-baseline leg of the benchmark may import it.  It shares no code with
the HIP path (no kernels, headers, tables or helpers) and imports nothing
from it; the two meet only through the seeded inputs of ``synth``.

Contents
  codecs  -- bf16 and OCP e4m3fn, from their bit-level definitions
  ops     -- add+RMSNorm, linear, SiLU-gated MLP, RoPE, FP8 KV quantiser,
             causal GQA attention, logprob, MoE top-K with ties and combine,
             acceptance statistics (max/mean/std diff and k3 KL)
  model   -- the decoder forward over any chunking of a sequence
  sparse  -- index scores, Top-K with a fixed tie rule in position order,
             attention over the selected keys
  ssd     -- the Mamba-2-style selective state-space recurrence
  backward -- gradients of add+RMSNorm, the SiLU-gated MLP, linear layers and
             the lm_head logprob (roundings straight-through)

Every function is pinned by a CPU test (tests/test_oracle_*.py) against
something other than itself: library routines, closed forms, brute force or
invariants.  The full-model forward is pinned only through its parts plus
invariants (causality, per-sequence independence, prefill == chunked ==
token-by-token decode); the pages print no logprob values to compare with.
"""
from . import backward, codecs, ops, model, sparse, ssd  # noqa: F401
