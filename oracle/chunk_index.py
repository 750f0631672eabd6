"""Chunk selection by key summaries, written out plainly (test infrastructure only).

CISA abstract (fugumt page 4), sentences 3-5: KV chunks of fixed size are selected with
compact summaries of the existing keys, one indexing query per KV group scores them, and the
selected chunks are shared by every query of the group (QShare reuses the selection across
adjacent queries).  Readings where the abstract is silent:
  * a chunk is ``chunk`` consecutive key tokens, n_chunks = ceil(Nk / chunk); the last chunk
    may be short;
  * its summary is the mean of its keys (float64 here), per (batch, KV group);
  * the indexing query of (batch, KV group g) is the mean, over the group's query heads,
    of the query at row ``query_index`` (the last query row for a prefill block);
  * score = <summary, indexing query>; the ``topk`` highest scores are kept, ties to the
    lower chunk index; the result lists chunk ids in ascending order.
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_to_f64


def _widen(x):
    x = np.asarray(x)
    return bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def chunk_summaries(k, chunk: int) -> np.ndarray:
    """Mean key of every chunk: k [B, Nk, Hkv, d] -> float64 [B, Hkv, n_chunks, d]."""
    kf = _widen(k)
    B, Nk, Hkv, d = kf.shape
    n = -(-Nk // chunk)
    out = np.zeros((B, Hkv, n, d))
    for c in range(n):
        t0, t1 = c * chunk, min(Nk, (c + 1) * chunk)
        out[:, :, c, :] = kf[:, t0:t1].mean(axis=1)
    return out


def indexing_queries(q, Hkv: int, query_index: int) -> np.ndarray:
    """One indexing query per (batch, KV group): the mean over the group's query heads of
    Q at row ``query_index``.  q [B, Nq, Hq, d] -> float64 [B, Hkv, d]."""
    qf = _widen(q)
    B, Nq, Hq, d = qf.shape
    grp = Hq // Hkv
    return qf[:, query_index].reshape(B, Hkv, grp, d).mean(axis=2)


def chunk_scores(q, k, chunk: int, Hkv: int, query_index: int) -> np.ndarray:
    """score[b, g, c] = <summary[b, g, c], indexing query[b, g]> in float64."""
    return np.einsum("bgcd,bgd->bgc", chunk_summaries(k, chunk), indexing_queries(q, Hkv, query_index))


def select_chunks(scores: np.ndarray, topk: int) -> np.ndarray:
    """The topk best chunks of every (b, g) row, ties to the lower index, ascending ids:
    [B, Hkv, n] -> int32 [B, Hkv, topk]."""
    B, G, n = scores.shape
    out = np.empty((B, G, topk), dtype=np.int32)
    for b in range(B):
        for g in range(G):
            order = sorted(range(n), key=lambda c: (-scores[b, g, c], c))
            out[b, g] = sorted(order[:topk])
    return out
