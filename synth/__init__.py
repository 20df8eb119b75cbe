"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package only *produces inputs*: loop-correlated keys/values, queries,
codebook fixtures, page tables and sequence lengths.  It computes none of the
quantity under test (no encoding of a cache, no dequantisation, no RoPE, no
attention), so neither side of a parity check can lean on it for its answer.
"""
from .gen import *  # noqa: F401,F403
