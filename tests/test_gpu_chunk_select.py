"""GPU parity of the chunk selection (bsattn_chunk_select) against the float64 oracle.

Summaries: float32 sums of bf16 keys against float64 means, max-abs error <= 1e-5 (a chunk
of 64 values of magnitude ~4 carries fp32 rounding of a few 1e-7).  Selection: a top-k
decided on float32 scores may differ from the float64 one only among near-ties at the
cut.  With s_k the oracle's k-th best score and eps = 1e-5 * max_c sum_e |summary_ce * iq_e|
(a bound on the float32 score error), every chunk scoring above s_k + eps must be selected,
none scoring below s_k - eps may be, and the ids must be topk distinct ascending values.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_fwd_amd as bs
from oracle.chunk_index import chunk_summaries, indexing_queries, select_chunks
from workloads.configs import make_chunk_gqa, normal_bf16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def check_unit(summ_gpu, sel_gpu, q, k, chunk, topk, query_index, label):
    """q [1, Nq, grp, d], k [1, Nk, 1, d]: one (batch, KV group)."""
    summ = chunk_summaries(k, chunk)[0, 0]
    iq = indexing_queries(q, 1, query_index)[0, 0]
    err = np.abs(summ_gpu - summ).max()
    assert err <= 1e-5, f"{label}: summary error {err}"
    s = summ @ iq
    sk = np.sort(s)[::-1][topk - 1]
    eps = 1e-5 * np.abs(summ * iq[None, :]).sum(axis=1).max()
    sel = np.asarray(sel_gpu)
    assert sel.shape == (topk,) and np.all(np.diff(sel) > 0) and sel.min() >= 0 and sel.max() < s.shape[0]
    must = np.nonzero(s > sk + eps)[0]
    never = np.nonzero(s < sk - eps)[0]
    assert np.isin(must, sel).all(), f"{label}: a clearly selected chunk is missing"
    assert not np.isin(never, sel).any(), f"{label}: a clearly unselected chunk is present"
    exact = np.array_equal(sel, select_chunks(s[None, None], topk)[0, 0])
    _say(f"{label}: summary err {err:.2e}; selection {'equal' if exact else 'equal up to near-ties'}")


# chunk counts n: 301, 136, 16, then the selection's edge sizes -- 8192 (the maximum: eight
# keys per thread), 1025 (two per thread for some threads) and a single short chunk
@pytest.mark.parametrize("d,Nk,chunk,topk,Hq,Hkv", [(128, 64 * 300 + 17, 64, 120, 8, 2), (64, 5000, 37, 50, 4, 4),
                                                 (128, 1024, 64, 16, 2, 1), (128, 8 * 8192, 8, 3000, 4, 2),
                                                 (64, 16 * 1025, 16, 1000, 2, 1), (128, 20, 64, 1, 2, 2)])
def test_chunk_select_small(d, Nk, chunk, topk, Hq, Hkv):
    rng = np.random.default_rng(d + Nk)
    B, Nq = 2, 33
    q = normal_bf16(rng, (B, Nq, Hq, d))
    k = normal_bf16(rng, (B, Nk, Hkv, d))
    summ, chunks = bs.chunk_select(_dev(q), _dev(k), Hkv, chunk, topk)
    torch.cuda.synchronize()
    summ = summ.cpu().numpy()
    chunks = chunks.cpu().numpy()
    grp = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            check_unit(summ[b, g], chunks[b, g], q[b:b + 1, :, g * grp:(g + 1) * grp], k[b:b + 1, :, g:g + 1],
                       chunk, topk, Nq - 1, f"b{b} g{g}")


def test_chunk_select_every_chunk():
    # topk = n: every chunk is selected, in ascending order
    rng = np.random.default_rng(11)
    q = normal_bf16(rng, (1, 9, 2, 128))
    k = normal_bf16(rng, (1, 64 * 100 - 5, 1, 128))
    _, chunks = bs.chunk_select(_dev(q), _dev(k), 1, 64, 100)
    torch.cuda.synchronize()
    assert np.array_equal(chunks.cpu().numpy()[0, 0], np.arange(100))


@pytest.mark.parametrize("topk", [1, 150, 300, 467, 699])
def test_chunk_select_exact_ties(topk):
    # chunk c holds key pattern c % 3: three exactly tied score levels (identical chunks
    # give bitwise identical float32 and float64 scores), so the selection at the cut must
    # take the lowest ids of the tied level, exactly as the oracle does
    rng = np.random.default_rng(12)
    chunk, n, d = 16, 700, 128
    pats = normal_bf16(rng, (3, chunk, d))
    k = np.concatenate([pats[c % 3] for c in range(n)], axis=0)[None, :, None, :]
    q = normal_bf16(rng, (1, 5, 4, d))
    summ, chunks = bs.chunk_select(_dev(q), _dev(k), 1, chunk, topk)
    torch.cuda.synchronize()
    sel = chunks.cpu().numpy()[0, 0]
    summ_ref, iq = chunk_summaries(k, chunk)[0, 0], indexing_queries(q, 1, 4)[0, 0]
    s = np.array([summ_ref[c] @ iq for c in range(n)])  # one dot per chunk: tied chunks tie exactly
    assert len(np.unique(s)) == 3
    ref = select_chunks(s[None, None], topk)[0, 0]
    _say(f"ties topk={topk}: selected {len(sel)}, first {sel[:4]}")
    assert np.array_equal(sel, ref)


def test_chunk_select_long_prefill_sampled():
    # the chunk-indexed GQA prefill shape: 4 x 262,144 keys, 8 KV groups of 8 query heads,
    # 64-token chunks, top-2048; two (batch, group) units checked against the oracle
    # (only the drawn Q and K are used here: a placeholder selection spares the oracle's)
    w = make_chunk_gqa("chunk-gqa", 5, B=4, Hq=64, Hkv=8, d=128, Nk=262144, Nq=2048, chunk=64, topk=2048,
                       chunk_select=lambda w_, c, t: np.tile(np.arange(t, dtype=np.int32), (w_.B * w_.Hkv, 1)))
    summ, chunks = bs.chunk_select(_dev(w.q), _dev(w.k), w.Hkv, 64, 2048)
    torch.cuda.synchronize()
    summ = summ.cpu().numpy()
    chunks = chunks.cpu().numpy()
    for b, g in ((0, 0), (3, 5)):
        check_unit(summ[b, g], chunks[b, g], w.q[b:b + 1, :, g * 8:(g + 1) * 8], w.k[b:b + 1, :, g:g + 1], 64, 2048,
                   w.Nq - 1, f"prefill b{b} g{g}")
