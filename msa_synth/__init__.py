"""Seeded synthetic inputs for the MSA hot path.

This module is the one place both sides draw their inputs from: the CPU
oracle (through the tests and the bench's CPU leg) and the HIP library
(through the tests and the bench).  It holds none of the method's arithmetic:
no RoPE, no pooling, no cosine, no top-k, no softmax.  It makes bits:

* ``normal_f32`` / ``normal_bf16``: standard normals from NumPy's PCG64,
  keyed by (seed, stream), rounded once to the storage dtype.
* ``counter_bf16``: a counter-based generator for banks too large to hold on
  the host.  Element i of stream s is SplitMix64 (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014) output
  number i+1 from a state keyed by (seed, s); four 6-bit fields of it are
  summed, centred and divided by 32, which is exact in bfloat16.  The same
  definition is implemented by the HIP fill kernel in ``fill.hip``; tests
  check the two bit for bit.
* document-length recipes and offset prefix sums, and the planting recipe
  that makes a few documents relevant to a query.
"""

from .gen import (normal_f32, normal_bf16, f32_to_bf16_bits, bf16_bits_to_f32,
                  splitmix64_key, counter_bf16, counter_f32,
                  uniform_lengths, lognormal_lengths, prefix_offsets,
                  ceil_chunk_offsets, planted_rows, pick_planted)

__all__ = [
    "normal_f32", "normal_bf16", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "splitmix64_key", "counter_bf16", "counter_f32",
    "uniform_lengths", "lognormal_lengths", "prefix_offsets",
    "ceil_chunk_offsets", "planted_rows", "pick_planted",
]
