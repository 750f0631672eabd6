"""Seeded synthetic inputs for exact block-sparse attention.

This module is shared by the oracle-side tests and by the GPU path's tests and
benchmark.  It produces *inputs only*: token layouts (blocks as contiguous slot
ranges, with an optional slot->token permutation), block selections, and bf16
Q/K/V tensors.  It performs none of the attention arithmetic and none of the
planning (paging, tile routing, pair counting).

Sources for the shapes (KPage abstract, zhuanzhiai page 1; CISA abstract,
fugumt page 4):
  * KPage abstract, sentences 1-3: 3D video token layouts whose blocks are
    partially occupied; 16-row K/V pages.
  * CISA abstract, sentences 3-5: fixed-size KV chunks selected by compact key
    summaries, one indexing query per KV group, shared across the group's
    queries (QShare across adjacent prefill queries).
"""
from .configs import Workload, make, CONFIG_NAMES, bf16_bits_from_f32, f32_from_bf16_bits  # noqa: F401
