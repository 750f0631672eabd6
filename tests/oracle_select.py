"""Chunk selection of the chunk-indexed workloads, taken from the float64 oracle.

The workload generator draws Q and K and asks its caller for the selection; the tests
pass this function, so both the GPU path and the oracle attention see the oracle's
selection (CISA abstract, fugumt page 4, sentences 3-5).  Results are cached per
(workload name, seed, chunk, top-k) within a test process: the full-size selection widens
all of K to float64.
"""
from __future__ import annotations

import numpy as np

from oracle.chunk_index import chunk_scores, select_chunks

_cache = {}


def oracle_chunk_select(w, chunk: int, topk: int) -> np.ndarray:
    key = (w.name, w.seed, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, chunk, topk)
    if key not in _cache:
        sel = select_chunks(chunk_scores(w.q, w.k, chunk, w.Hkv, w.Nq - 1), topk)
        _cache[key] = np.asarray(sel, dtype=np.int32).reshape(w.B * w.Hkv, topk)
    return _cache[key]
