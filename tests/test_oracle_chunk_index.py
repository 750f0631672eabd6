"""Pins for the chunk-selection oracle (CPU only).

  * closed form: keys constant within each chunk and equal query heads make the summary
    and the indexing query known exactly, so every score and the selection are known;
  * ties: equal scores select the lowest chunk ids; topk = n_chunks selects all;
  * a short last chunk is averaged over its own keys only (pure-Python loops);
  * brute force: scalar loops for summaries, indexing query, dot product and a full
    ranking on a tiny random case.
"""
import math

import numpy as np

from oracle.chunk_index import chunk_summaries, indexing_queries, chunk_scores, select_chunks
from workloads.configs import normal_bf16


def test_closed_form_scores_and_selection():
    B, Hkv, grp, d, chunk, n = 2, 3, 4, 8, 5, 9
    alpha = np.array([[[3.0, -1.0, 7.0, 0.5, 2.0, 9.0, -4.0, 6.0, 1.0]] * Hkv] * B)
    alpha[1, 2] = alpha[1, 2][::-1]
    k = np.zeros((B, n * chunk, Hkv, d))
    for b in range(B):
        for g in range(Hkv):
            for c in range(n):
                k[b, c * chunk:(c + 1) * chunk, g, 0] = alpha[b, g, c]
    q = np.zeros((B, 6, Hkv * grp, d))
    q[:, 5, :, 0] = 2.0      # every head of the last row: 2 e_0, so the indexing query is 2 e_0
    q[:, 5, :, 1] = 99.0     # summaries have 0 in column 1: no effect on the score
    s = chunk_scores(q, k, chunk, Hkv, 5)
    np.testing.assert_array_equal(s, 2.0 * alpha)
    sel = select_chunks(s, 3)
    np.testing.assert_array_equal(sel[0, 0], [2, 5, 7])        # 7, 9, 6 are the three largest
    np.testing.assert_array_equal(sel[1, 2], [1, 3, 6])        # the reversed row


def test_ties_and_full_selection():
    s = np.zeros((1, 1, 10))
    np.testing.assert_array_equal(select_chunks(s, 4)[0, 0], [0, 1, 2, 3])
    s[0, 0, 7] = 1.0
    np.testing.assert_array_equal(select_chunks(s, 4)[0, 0], [0, 1, 2, 7])
    r = np.random.default_rng(0).standard_normal((2, 3, 10))
    np.testing.assert_array_equal(select_chunks(r, 10), np.broadcast_to(np.arange(10), (2, 3, 10)))


def test_short_last_chunk_and_brute_force():
    rng = np.random.default_rng(5)
    B, Nk, Hkv, grp, d, chunk, Nq = 2, 23, 2, 3, 4, 5, 4
    k = normal_bf16(rng, (B, Nk, Hkv, d))
    q = normal_bf16(rng, (B, Nq, Hkv * grp, d))
    kf = (k.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    summ = chunk_summaries(k, chunk)
    iq = indexing_queries(q, Hkv, 2)
    n = math.ceil(Nk / chunk)
    assert summ.shape == (B, Hkv, n, d)
    for b in range(B):
        for g in range(Hkv):
            qv = [sum(qf[b, 2, g * grp + h, e] for h in range(grp)) / grp for e in range(d)]
            for e in range(d):
                assert abs(iq[b, g, e] - qv[e]) < 1e-15
            sc = []
            for c in range(n):
                rows = list(range(c * chunk, min(Nk, (c + 1) * chunk)))
                m = [sum(kf[b, t, g, e] for t in rows) / len(rows) for e in range(d)]
                for e in range(d):
                    assert abs(summ[b, g, c, e] - m[e]) < 1e-15
                sc.append(sum(m[e] * qv[e] for e in range(d)))
            s = chunk_scores(q, k, chunk, Hkv, 2)[b, g]
            assert max(abs(s[c] - sc[c]) for c in range(n)) < 1e-12
            best = []
            for _ in range(3):  # three rounds of "largest remaining, lowest index on ties"
                cand = [c for c in range(n) if c not in best]
                top = max(sc[c] for c in cand)
                best.append(min(c for c in cand if sc[c] == top))
            assert list(select_chunks(s[None, None], 3)[0, 0]) == sorted(best)
