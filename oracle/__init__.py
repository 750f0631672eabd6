"""CPU oracle for exact block-sparse softmax attention (test infrastructure only).

This package is the slow, plainly written reference that the GPU path is checked
against.  It is imported only by ``tests/``, by ``__graft_entry__.smoke()`` and by the
CPU-baseline leg of ``bench.py``; the product path never calls it and must fail
loudly when its HIP library is missing.

Contents
  attention.py  masked dense softmax attention in float64 (numpy): the full masked
                score matrix, -inf outside the sparse graph, softmax, times V; plus a
                pure-Python scalar brute force for tiny inputs; and the gradients of
                that function (dQ, dK, dV) for an upstream gradient of O.
  planner.py    the page / tile plan: 16-row K/V pages owned by one block, Q-block
                routing between 128x128 and 64x256 tiles, per-(unit, Q block) page
                lists and the useful / physical query-key pair counts; the backward
                tables (Q pages, owned tiles of each side, Q page lists per
                (unit, K block)).
  chunk_index.py  chunk selection: mean-key chunk summaries, one indexing query per
                KV group, top-k chunks (CISA abstract, sentences 3-5).

Sources (cited by page title and passage):
  * KPage abstract (zhuanzhiai page 1): sentence 2 (16-row K/V pages of valid tokens,
    packed across block boundaries into large tiles while loading), sentence 3 (Q
    blocks routed between 64x256 and 128x128 tiles), sentence 4 (pages belong to one
    K/V block and masking is exact: only the selected graph's pairs count), sentence 7
    (physical vs useful query-key pairs).
  * CISA abstract (fugumt page 4): sentences 3-5 (KV chunks selected per KV group and
    shared by the group's queries) -- the selection is an input here.
  * FlashAttention entries of the related-paper lists (scifaro pages 2 and 3): exact
    softmax attention; its log-sum-exp output convention.

Parity status: every function here is pinned by tests that do not re-use its code
(closed forms, brute force, library routines, invariants); see tests/test_oracle_*.py.
"""
from .attention import (  # noqa: F401
    bf16_to_f64, token_block_map, selection_unit, selected_blocks, token_mask,
    masked_attention, brute_force_attention, useful_pairs, masked_attention_bwd, masked_attention_bwd_w,
)
from .planner import Plan, build_plan, BwdPlan, build_bwd_plan  # noqa: F401
from .chunk_index import chunk_summaries, indexing_queries, chunk_scores, select_chunks  # noqa: F401
