"""Masked dense softmax attention in float64 -- the definition, written out.

Test infrastructure only (see the package docstring).

What is computed (KPage abstract, sentences 2 and 4: packing changes only how pairs are
grouped into tiles and masking is exact, so the result is plain masked softmax attention):

  For batch b, query head h with KV head g = h // (Hq / Hkv), query token i and key
  token j, the pair (i, j) is in the graph iff the K block holding j is in the
  selected set of the Q block holding i for the selection unit of (b, h), and, for a
  causal problem, key position j <= query position q_pos0 + i.
      S_ij   = scale * <Q[b, i, h, :], K[b, j, g, :]>   (pairs outside the graph: -inf)
      m_i    = max_j S_ij
      O_i    = sum_j exp(S_ij - m_i) V[b, j, g, :] / sum_j exp(S_ij - m_i)
      LSE_i  = m_i + ln sum_j exp(S_ij - m_i)             (natural log)
  A row with no key in the graph has O_i = 0 and LSE_i = -inf.

The score matrix is materialised in row chunks of the full key width: a chunk gives
exactly the rows the whole matrix would, with bounded memory.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

ROW_CHUNK = 256


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of a float32)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def token_block_map(offsets: np.ndarray, perm: Optional[np.ndarray], n_tokens: int) -> np.ndarray:
    """Block id of every token.  Slots [offsets[k], offsets[k+1]) form block k; slot s holds
    token perm[s] (token s when perm is None).  The layout must cover every token once."""
    offsets = np.asarray(offsets, dtype=np.int64)
    if offsets[0] != 0 or offsets[-1] != n_tokens or np.any(np.diff(offsets) < 0):
        raise ValueError("layout offsets must rise from 0 to the token count")
    blk = np.full(n_tokens, -1, dtype=np.int64)
    slots_block = np.repeat(np.arange(offsets.shape[0] - 1), np.diff(offsets))
    tokens = np.arange(n_tokens) if perm is None else np.asarray(perm, dtype=np.int64)
    if perm is not None and (tokens.shape[0] != n_tokens or np.any(np.sort(tokens) != np.arange(n_tokens))):
        raise ValueError("perm must be a permutation of the tokens")
    blk[tokens] = slots_block
    return blk


def selection_unit(b: int, h: int, B: int, Hq: int, Hkv: int, sel_nb: int, sel_nh: int) -> int:
    """Index of the selection unit used by (batch b, query head h).
    sel_nb is 1 (shared over batch) or B; sel_nh is 1 (shared over heads), Hkv (one per KV
    group, shared by that group's query heads -- CISA abstract, sentence 4) or Hq."""
    ub = b if sel_nb == B else 0
    if sel_nh == Hq:
        uh = h
    elif sel_nh == Hkv:
        uh = h // (Hq // Hkv)
    elif sel_nh == 1:
        uh = 0
    else:
        raise ValueError("sel_nh must be 1, Hkv or Hq")
    if sel_nb not in (1, B):
        raise ValueError("sel_nb must be 1 or B")
    return ub * sel_nh + uh


def selected_blocks(row_ptr: np.ndarray, kblk: np.ndarray, row: int, n_kblocks: int) -> np.ndarray:
    """The selected K-block set of one (unit, Q block) row: sorted, duplicates removed."""
    s = np.asarray(kblk[row_ptr[row]:row_ptr[row + 1]], dtype=np.int64)
    if s.size and (s.min() < 0 or s.max() >= n_kblocks):
        raise ValueError("selected block id out of range")
    return np.unique(s)


def token_mask(bq: np.ndarray, bk: np.ndarray, row_ptr, kblk, unit: int, n_qblocks: int, n_kblocks: int,
               q_tokens: np.ndarray, causal: bool, q_pos0: int) -> np.ndarray:
    """Boolean mask [len(q_tokens), Nk]: True where (query token, key token) is in the graph."""
    member = np.zeros((n_qblocks, n_kblocks), dtype=bool)
    for qb in np.unique(bq[q_tokens]):
        member[qb, selected_blocks(row_ptr, kblk, unit * n_qblocks + int(qb), n_kblocks)] = True
    m = member[bq[q_tokens]][:, bk]
    if causal:
        kpos = np.arange(bk.shape[0], dtype=np.int64)
        qpos = q_pos0 + np.asarray(q_tokens, dtype=np.int64)
        m &= kpos[None, :] <= qpos[:, None]
    return m


def masked_attention(q, k, v, q_offsets, q_perm, k_offsets, k_perm, sel_nb, sel_nh, sel_row_ptr, sel_kblk,
                     scale: float, causal: bool = False, q_pos0: int = 0,
                     rows: Optional[Sequence[Tuple[int, int, np.ndarray]]] = None):
    """Exact masked softmax attention in float64.

    q: [B, Nq, Hq, d], k and v: [B, Nk, Hkv, d] as bf16 bits (uint16) or float arrays.
    Returns (O float64 [B, Nq, Hq, d], LSE float64 [B, Hq, Nq]) when ``rows`` is None.
    With ``rows`` = [(b, h, query_tokens), ...] returns a list of (O_rows, LSE_rows).
    """
    def widen(x):
        x = np.asarray(x)
        return bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)

    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    bq = token_block_map(q_offsets, q_perm, Nq)
    bk = token_block_map(k_offsets, k_perm, Nk)
    nqb, nkb = len(q_offsets) - 1, len(k_offsets) - 1

    def one(b, h, toks):
        g = h // (Hq // Hkv)
        unit = selection_unit(b, h, B, Hq, Hkv, sel_nb, sel_nh)
        kf = widen(k[b, :, g, :])
        vf = widen(v[b, :, g, :])
        o = np.zeros((len(toks), d))
        lse = np.full(len(toks), -np.inf)
        for c0 in range(0, len(toks), ROW_CHUNK):
            t = np.asarray(toks[c0:c0 + ROW_CHUNK], dtype=np.int64)
            qf = widen(q[b, t, h, :])
            s = scale * (qf @ kf.T)
            msk = token_mask(bq, bk, sel_row_ptr, sel_kblk, unit, nqb, nkb, t, causal, q_pos0)
            s[~msk] = -np.inf
            mx = s.max(axis=1)
            live = mx > -np.inf
            p = np.zeros_like(s)
            p[live] = np.exp(s[live] - mx[live, None])
            l = p.sum(axis=1)
            o[c0:c0 + len(t)][live] = (p[live] @ vf) / l[live, None]
            lse[c0:c0 + len(t)][live] = mx[live] + np.log(l[live])
        return o, lse

    if rows is not None:
        return [one(b, h, np.asarray(t)) for (b, h, t) in rows]
    O = np.zeros((B, Nq, Hq, d))
    L = np.full((B, Hq, Nq), -np.inf)
    allq = np.arange(Nq)
    for b in range(B):
        for h in range(Hq):
            o, lse = one(b, h, allq)
            O[b, :, h, :] = o
            L[b, h, :] = lse
    return O, L


def masked_attention_w(w, rows=None):
    """Convenience wrapper for any object carrying the problem's fields."""
    return masked_attention(w.q, w.k, w.v, w.q_offsets, w.q_perm, w.k_offsets, w.k_perm, w.sel_nb, w.sel_nh,
                            w.sel_row_ptr, w.sel_kblk, w.scale, w.causal, w.q_pos0, rows=rows)


def useful_pairs(q_offsets, q_perm, k_offsets, k_perm, B, Hq, Hkv, sel_nb, sel_nh, sel_row_ptr, sel_kblk,
                 causal=False, q_pos0=0) -> int:
    """Number of (batch, head, query, key) pairs in the graph, i.e. the mask's nonzeros,
    summed block by block: each (query, selected key) combination counted once."""
    Nq = int(q_offsets[-1])
    Nk = int(k_offsets[-1])
    nqb, nkb = len(q_offsets) - 1, len(k_offsets) - 1
    ktok_sorted = []
    for kb in range(nkb):
        sl = np.arange(k_offsets[kb], k_offsets[kb + 1], dtype=np.int64)
        toks = sl if k_perm is None else np.asarray(k_perm, dtype=np.int64)[sl]
        ktok_sorted.append(np.sort(toks))
    ksize = np.diff(np.asarray(k_offsets, dtype=np.int64))

    def row_pairs(unit, qb):
        sel = selected_blocks(sel_row_ptr, sel_kblk, unit * nqb + qb, nkb)
        nq = int(q_offsets[qb + 1] - q_offsets[qb])
        if nq == 0 or sel.size == 0:
            return 0
        if not causal:
            return nq * int(ksize[sel].sum())
        sl = np.arange(q_offsets[qb], q_offsets[qb + 1], dtype=np.int64)
        qtok = sl if q_perm is None else np.asarray(q_perm, dtype=np.int64)[sl]
        qpos = q_pos0 + qtok
        return sum(int(np.searchsorted(ktok_sorted[kb], qpos, side="right").sum()) for kb in sel)

    per_unit = {}  # heads that share a selection unit have the same count
    total = 0
    for b in range(B):
        for h in range(Hq):
            unit = selection_unit(b, h, B, Hq, Hkv, sel_nb, sel_nh)
            if unit not in per_unit:
                per_unit[unit] = sum(row_pairs(unit, qb) for qb in range(nqb))
            total += per_unit[unit]
    return total


# ----------------------------------------------------------------------------
# pure-Python brute force for tiny inputs
# ----------------------------------------------------------------------------
def brute_force_attention(q, k, v, q_offsets, q_perm, k_offsets, k_perm, sel_nb, sel_nh, sel_row_ptr, sel_kblk,
                          scale, causal=False, q_pos0=0):
    """Scalar loops with math.exp, for inputs of a few dozen tokens.  Block membership is
    found by scanning the layout slots and the selection list directly; nothing is
    shared with :func:`masked_attention` but the bf16 widening."""
    qf, kf, vf = (bf16_to_f64(x) if np.asarray(x).dtype == np.uint16 else np.asarray(x, np.float64)
                  for x in (q, k, v))
    B, Nq, Hq, d = qf.shape
    Nk, Hkv = kf.shape[1], kf.shape[2]
    nqb, nkb = len(q_offsets) - 1, len(k_offsets) - 1

    def block_of(offsets, perm, tok):
        for blk in range(len(offsets) - 1):
            for s in range(int(offsets[blk]), int(offsets[blk + 1])):
                if (s if perm is None else int(perm[s])) == tok:
                    return blk
        raise ValueError("token not in layout")

    O = [[[[0.0] * d for _ in range(Hq)] for _ in range(Nq)] for _ in range(B)]
    L = [[[-math.inf] * Nq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h * Hkv // Hq
            ub = b if sel_nb == B else 0
            uh = h if sel_nh == Hq else (g if sel_nh == Hkv else 0)
            unit = ub * sel_nh + uh
            for i in range(Nq):
                qb = block_of(q_offsets, q_perm, i)
                row = unit * nqb + qb
                chosen = [int(x) for x in sel_kblk[int(sel_row_ptr[row]):int(sel_row_ptr[row + 1])]]
                keys = []
                for j in range(Nk):
                    if block_of(k_offsets, k_perm, j) in chosen and (not causal or j <= q_pos0 + i):
                        keys.append(j)
                if not keys:
                    continue
                sc = []
                for j in keys:
                    acc = 0.0
                    for e in range(d):
                        acc += qf[b, i, h, e] * kf[b, j, g, e]
                    sc.append(scale * acc)
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                tot = math.fsum(w)
                for e in range(d):
                    O[b][i][h][e] = math.fsum(w[t] * vf[b, keys[t], g, e] for t in range(len(keys))) / tot
                L[b][h][i] = m + math.log(tot)
    return np.array(O), np.array(L)


# ----------------------------------------------------------------------------
# backward: gradients of the same masked softmax attention
# ----------------------------------------------------------------------------
# KPage abstract, sentence 4: the backward works on the same selected pairs (pages owned by
# one K/V block, exact masking), so the gradients are those of the function above.  With
# P^_ij = exp(S_ij - LSE_i) (zero outside the graph and on rows without keys) and an
# upstream gradient dO of O, the chain rule through O = P^ V and the row softmax gives
#     D_i   = sum_e dO_ie O_ie
#     dV_j  = sum over query heads of the KV group, sum_i P^_ij dO_i
#     dS_ij = P^_ij (dO_i . V_j - D_i)
#     dQ_i  = scale sum_j dS_ij K_j
#     dK_j  = scale sum over query heads of the group, sum_i dS_ij Q_i
# D uses the exact O of the forward oracle.

def _widen(x):
    x = np.asarray(x)
    return bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def _bwd_head_chunk(qf, kf, vf, dof, t, bq, bk, row_ptr, kblk, unit, nqb, nkb, scale, causal, q_pos0):
    """Rows t of one (batch, query head): the masked probabilities P^ [len(t), Nk] and
    dS [len(t), Nk] over the full key width."""
    s = scale * (qf[t] @ kf.T)
    msk = token_mask(bq, bk, row_ptr, kblk, unit, nqb, nkb, t, causal, q_pos0)
    s[~msk] = -np.inf
    mx = s.max(axis=1)
    live = mx > -np.inf
    p = np.zeros_like(s)
    p[live] = np.exp(s[live] - mx[live, None])
    l = p.sum(axis=1)
    p[live] /= l[live, None]
    o = p @ vf
    D = np.sum(dof[t] * o, axis=1)
    dP = dof[t] @ vf.T
    dS = p * (dP - D[:, None])
    return p, dS


def masked_attention_bwd(q, k, v, do, q_offsets, q_perm, k_offsets, k_perm, sel_nb, sel_nh, sel_row_ptr,
                         sel_kblk, scale: float, causal: bool = False, q_pos0: int = 0,
                         q_rows: Optional[Sequence[Tuple[int, int, np.ndarray]]] = None,
                         k_rows: Optional[Sequence[Tuple[int, int, np.ndarray]]] = None):
    """Gradients (dQ, dK, dV) of masked softmax attention in float64 for the upstream
    gradient ``do`` of O (same shape as Q).

    With neither ``q_rows`` nor ``k_rows`` returns full arrays dQ [B, Nq, Hq, d] and
    dK, dV [B, Nk, Hkv, d].  With ``q_rows`` = [(b, h, query tokens), ...] and/or
    ``k_rows`` = [(b, g, key tokens), ...] returns (list of dQ rows, list of (dK rows,
    dV rows)); a key's rows sum over every query head of KV group g and over every query
    in the graph with it, whose full rows are computed for their softmax statistics.
    """
    B, Nq, Hq, d = np.asarray(q).shape
    Nk, Hkv = np.asarray(k).shape[1], np.asarray(k).shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    grp = Hq // Hkv
    bq = token_block_map(q_offsets, q_perm, Nq)
    bk = token_block_map(k_offsets, k_perm, Nk)
    nqb, nkb = len(q_offsets) - 1, len(k_offsets) - 1
    heads = {}

    def head(b, h):
        if (b, h) not in heads:
            g = h // grp
            heads.clear()
            heads[(b, h)] = (_widen(q[b, :, h, :]), _widen(k[b, :, g, :]), _widen(v[b, :, g, :]),
                             _widen(do[b, :, h, :]), selection_unit(b, h, B, Hq, Hkv, sel_nb, sel_nh))
        return heads[(b, h)]

    def rows_dq(b, h, toks):
        qf, kf, vf, dof, unit = head(b, h)
        out = np.zeros((len(toks), d))
        for c0 in range(0, len(toks), ROW_CHUNK):
            t = np.asarray(toks[c0:c0 + ROW_CHUNK], dtype=np.int64)
            _, dS = _bwd_head_chunk(qf, kf, vf, dof, t, bq, bk, sel_row_ptr, sel_kblk, unit, nqb, nkb, scale,
                                    causal, q_pos0)
            out[c0:c0 + len(t)] = scale * (dS @ kf)
        return out

    def keys_dkdv(b, g, ktoks, qtoks_of_head):
        ktoks = np.asarray(ktoks, dtype=np.int64)
        dk = np.zeros((len(ktoks), d))
        dv = np.zeros((len(ktoks), d))
        for h in range(g * grp, (g + 1) * grp):
            qf, kf, vf, dof, unit = head(b, h)
            toks = qtoks_of_head(h, unit)
            for c0 in range(0, len(toks), ROW_CHUNK):
                t = np.asarray(toks[c0:c0 + ROW_CHUNK], dtype=np.int64)
                p, dS = _bwd_head_chunk(qf, kf, vf, dof, t, bq, bk, sel_row_ptr, sel_kblk, unit, nqb, nkb, scale,
                                        causal, q_pos0)
                dv += p[:, ktoks].T @ dof[t]
                dk += scale * (dS[:, ktoks].T @ qf[t])
        return dk, dv

    allq = np.arange(Nq, dtype=np.int64)
    if q_rows is None and k_rows is None:
        dQ = np.zeros((B, Nq, Hq, d))
        dK = np.zeros((B, Nk, Hkv, d))
        dV = np.zeros((B, Nk, Hkv, d))
        for b in range(B):
            for h in range(Hq):
                qf, kf, vf, dof, unit = head(b, h)
                g = h // grp
                for c0 in range(0, Nq, ROW_CHUNK):
                    t = allq[c0:c0 + ROW_CHUNK]
                    p, dS = _bwd_head_chunk(qf, kf, vf, dof, t, bq, bk, sel_row_ptr, sel_kblk, unit, nqb, nkb,
                                            scale, causal, q_pos0)
                    dQ[b, t, h, :] = scale * (dS @ kf)
                    dV[b, :, g, :] += p.T @ dof[t]
                    dK[b, :, g, :] += scale * (dS.T @ qf[t])
        return dQ, dK, dV

    dq_out = [rows_dq(b, h, np.asarray(t)) for (b, h, t) in (q_rows or [])]

    def attending(ktoks):
        # queries whose graph row holds at least one of ktoks: their Q block selects a K block
        # of one of the keys (the causal bound is left to the full-row mask)
        kbs = np.unique(bk[np.asarray(ktoks, dtype=np.int64)])

        def f(h, unit):
            qbs = [qb for qb in range(nqb)
                   if np.intersect1d(selected_blocks(sel_row_ptr, sel_kblk, unit * nqb + qb, nkb), kbs).size]
            return allq[np.isin(bq, np.asarray(qbs, dtype=np.int64))]
        return f

    dkv_out = [keys_dkdv(b, g, np.asarray(t), attending(t)) for (b, g, t) in (k_rows or [])]
    return dq_out, dkv_out


def masked_attention_bwd_w(w, do, q_rows=None, k_rows=None):
    """Convenience wrapper for any object carrying the problem's fields."""
    return masked_attention_bwd(w.q, w.k, w.v, do, w.q_offsets, w.q_perm, w.k_offsets, w.k_perm, w.sel_nb,
                                w.sel_nh, w.sel_row_ptr, w.sel_kblk, w.scale, w.causal, w.q_pos0,
                                q_rows=q_rows, k_rows=k_rows)
