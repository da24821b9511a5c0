"""Seeded synthetic inputs for the five workloads (shared by tests, the
benchmark and the oracle checks).

This module draws random numbers, casts them to the storage formats with
torch's own conversions (round to nearest even; float8 e4m3fn), and places
rows into cache pages.  It holds none of the attention or RoPE arithmetic:
the RoPE table it builds is an *input* of the fused step (the kernels and the
oracle only read it), and prior cache contents are inputs written in the
storage format, as an earlier step would have left them.

Recipe (per workload, seed = workload number - 1):

* ``numpy.random.default_rng(seed)`` draws the lengths, then the physical page
  permutation;
* ``default_rng([seed, 1])`` draws the new tokens' q, k, v (float32 standard
  normal, in that order);
* ``default_rng([seed, 2, s])`` draws sequence s's prior cache rows (K then V,
  float32 standard normal) -- one stream per sequence, so any subset of
  sequences can be regenerated alone;
* QK-norm workloads divide each Q/K head vector by its root mean square in
  float64 before the cast (no epsilon, no weight);
* float8 prior rows: one scale per (token, kv head), float32 absmax / 448, and
  torch's e4m3fn cast of x / scale.

See ``synth.configs`` for the five workloads and the variants of the
prefill batch that exercise the band of keys and the RoPE layouts (M-RoPE
position streams: ``mrope_positions``).
"""

from .configs import (Workload, make, names, new_tokens, freqs_table, custom,  # noqa: F401
                      prior_rows, build_cache, sentinel_cache, mrope_positions)
from . import work  # noqa: F401
