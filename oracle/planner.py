"""The page / tile plan, written out rule by rule (test infrastructure only).

KPage abstract, sentence 2: keys and values are cut into 16-row pages of valid tokens,
and pages are packed across logical-block boundaries into large tiles while loading.
Sentence 3: Q blocks are routed between 64x256 and 128x128 tiles to cut query-side
padding.  Sentence 4: each page belongs to one K/V block and masking is exact, so only
the selected graph's pairs count.  Sentence 7: physical query-key pair capacity (what the
tiles hold, padding included) versus useful pairs (the graph's edges).

Readings of what the abstract leaves open (one per rule):
  R1 selection   a (unit, Q block) row selects a *set* of K blocks: sorted, deduplicated;
                 ids must be in range.
  R2 pages       a K block of n >= 1 slots has pages p = 0 .. ceil(n/16)-1, page p covering
                 slots [16p, min(16p+16, n)) of that block; an empty block has no pages.
  R3 tile shapes (Q rows x K columns) = 128x128 (8 pages per K tile) or 64x256 (16 pages).
  R4 Q routing   a Q block of n >= 1 rows gives floor(n/128) 128-row tiles in row order, then
                 for r = n mod 128: one 64-row tile if 0 < r <= 64, one 128-row tile if r > 64.
  R5 K tiles     a Q tile's page sequence is the pages of its selected blocks, block ascending
                 then page ascending, cut into ceil(n_pages / pages_per_tile) K tiles; only
                 the last K tile may hold empty page slots.  Nothing is pruned for causality.
  R6 counts      useful U = pairs in the graph (causal exclusions removed); physical
                 P = sum over (batch, head) and Q tiles of tile_rows * tile_cols * n_ktiles.

The fixed-tile baseline (``fixed_tiles=True``; the abstract's sentences 5 and 7 measure
packing and routing against NVIDIA BSA): R4 without the 64-row shape (ceil(n/128) 128-row
tiles per Q block) and R5 with every selected block starting a new K tile -- its pages are
followed by empty slots (page id -1) up to a multiple of 8 -- so a tile never holds pages
of two blocks.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from .attention import selected_blocks, selection_unit, useful_pairs

PAGE = 16
SHAPE_128x128 = 0
SHAPE_64x256 = 1
TILE_ROWS = {SHAPE_128x128: 128, SHAPE_64x256: 64}
TILE_COLS = {SHAPE_128x128: 128, SHAPE_64x256: 256}
PAGES_PER_KTILE = {SHAPE_128x128: 8, SHAPE_64x256: 16}


@dataclasses.dataclass
class Plan:
    # K pages (R2), in K-block order then page order; a page id is an index here
    page_kblock: np.ndarray
    page_slot0: np.ndarray      # absolute slot of the page's first row in the K layout
    page_nvalid: np.ndarray     # 1..16
    # Q tiles (R4), in Q-block order then row order
    qt_qblock: np.ndarray
    qt_row0: np.ndarray         # absolute slot of the tile's first row in the Q layout
    qt_rows: np.ndarray         # valid rows, 1..128 (or 1..64 for a 64-row tile)
    qt_shape: np.ndarray        # SHAPE_128x128 or SHAPE_64x256
    # page lists (R5) per (unit, Q block) row, CSR
    n_units: int
    pl_ptr: np.ndarray          # int64 [n_units * n_qblocks + 1]
    pl_pages: np.ndarray        # int32 page ids
    # counts (R6), over all (batch, head)
    useful: int
    physical: int
    n_ktiles: int
    useful_by_shape: tuple = (0, 0)
    physical_by_shape: tuple = (0, 0)

    @property
    def n_pages(self) -> int:
        return int(self.page_kblock.shape[0])

    @property
    def n_qtiles128(self) -> int:
        return int(np.sum(self.qt_shape == SHAPE_128x128))

    @property
    def n_qtiles64(self) -> int:
        return int(np.sum(self.qt_shape == SHAPE_64x256))


def build_plan(B, Hq, Hkv, q_offsets, q_perm, k_offsets, k_perm, sel_nb, sel_nh, sel_row_ptr, sel_kblk,
               causal=False, q_pos0=0, page_size=PAGE, fixed_tiles=False) -> Plan:
    if page_size != PAGE:
        raise ValueError("only 16-row pages are defined")
    nqb, nkb = len(q_offsets) - 1, len(k_offsets) - 1
    n_units = sel_nb * sel_nh
    if len(sel_row_ptr) != n_units * nqb + 1:
        raise ValueError("selection row_ptr has the wrong length")

    # R2: pages
    pk, ps, pn = [], [], []
    first_page = [0]
    for kb in range(nkb):
        s0, s1 = int(k_offsets[kb]), int(k_offsets[kb + 1])
        n = s1 - s0
        for p in range((n + PAGE - 1) // PAGE):
            pk.append(kb)
            ps.append(s0 + PAGE * p)
            pn.append(min(PAGE, n - PAGE * p))
        first_page.append(len(pk))

    # R4: Q routing
    qq, qr, qn, qs = [], [], [], []
    for qb in range(nqb):
        s0, s1 = int(q_offsets[qb]), int(q_offsets[qb + 1])
        n = s1 - s0
        full, r = divmod(n, 128)
        for t in range(full):
            qq.append(qb); qr.append(s0 + 128 * t); qn.append(128); qs.append(SHAPE_128x128)
        if 0 < r <= 64 and not fixed_tiles:
            qq.append(qb); qr.append(s0 + 128 * full); qn.append(r); qs.append(SHAPE_64x256)
        elif 0 < r <= 64:
            qq.append(qb); qr.append(s0 + 128 * full); qn.append(r); qs.append(SHAPE_128x128)
        elif r > 64:
            qq.append(qb); qr.append(s0 + 128 * full); qn.append(r); qs.append(SHAPE_128x128)

    # R1 + R5: page lists per (unit, Q block)
    pl_ptr = [0]
    pl = []
    for u in range(n_units):
        for qb in range(nqb):
            for kb in selected_blocks(sel_row_ptr, sel_kblk, u * nqb + qb, nkb):
                pl.extend(range(first_page[kb], first_page[kb + 1]))
                if fixed_tiles:
                    npg = first_page[kb + 1] - first_page[kb]
                    pl.extend([-1] * (-npg % PAGES_PER_KTILE[SHAPE_128x128]))
            pl_ptr.append(len(pl))
    pl_ptr = np.asarray(pl_ptr, dtype=np.int64)

    # R6: physical capacity and K-tile count over every (batch, head)
    physical = [0, 0]
    nkt = 0
    for b in range(B):
        for h in range(Hq):
            u = selection_unit(b, h, B, Hq, Hkv, sel_nb, sel_nh)
            for t in range(len(qq)):
                row = u * nqb + qq[t]
                npg = int(pl_ptr[row + 1] - pl_ptr[row])
                kt = -(-npg // PAGES_PER_KTILE[qs[t]])
                nkt += kt
                physical[qs[t]] += TILE_ROWS[qs[t]] * TILE_COLS[qs[t]] * kt
    useful = useful_pairs(q_offsets, q_perm, k_offsets, k_perm, B, Hq, Hkv, sel_nb, sel_nh,
                          sel_row_ptr, sel_kblk, causal, q_pos0)
    # useful pairs split by the shape of the Q tile that holds the query
    qshape = np.zeros(int(q_offsets[-1]), dtype=np.int64)
    for t in range(len(qq)):
        qshape[qr[t]:qr[t] + qn[t]] = qs[t]
    useful_sh = [0, 0]
    for sh in (0, 1):
        if not np.any(qshape == sh):
            continue
        # the same count restricted to queries of this shape: blocks cut down to those slots
        offs = np.asarray(q_offsets, dtype=np.int64)
        keep = np.nonzero(qshape == sh)[0]
        new_offs = np.searchsorted(keep, offs, side="left")
        sub_perm = None if q_perm is None else np.asarray(q_perm, dtype=np.int64)[keep]
        if sub_perm is None:
            sub_perm = keep
        useful_sh[sh] = _useful_subset(new_offs, sub_perm, k_offsets, k_perm, B, Hq, Hkv, sel_nb, sel_nh,
                                       sel_row_ptr, sel_kblk, causal, q_pos0)
    i32 = lambda a: np.asarray(a, dtype=np.int32)  # noqa: E731
    return Plan(page_kblock=i32(pk), page_slot0=i32(ps), page_nvalid=i32(pn),
                qt_qblock=i32(qq), qt_row0=i32(qr), qt_rows=i32(qn), qt_shape=i32(qs),
                n_units=n_units, pl_ptr=pl_ptr, pl_pages=i32(pl),
                useful=int(useful), physical=int(sum(physical)), n_ktiles=int(nkt),
                useful_by_shape=tuple(int(x) for x in useful_sh), physical_by_shape=tuple(int(x) for x in physical))


def _useful_subset(q_offsets, q_tokens, k_offsets, k_perm, B, Hq, Hkv, sel_nb, sel_nh, sel_row_ptr, sel_kblk,
                   causal, q_pos0):
    """Useful pairs of a subset of the query slots: ``q_offsets`` re-cut over the kept slots
    and ``q_tokens`` their tokens (positions for the causal test)."""
    nqb = len(q_offsets) - 1
    nkb = len(k_offsets) - 1

    def unit_pairs(u):
        tot = 0
        for qb in range(nqb):
            toks = np.asarray(q_tokens[q_offsets[qb]:q_offsets[qb + 1]], dtype=np.int64)
            if toks.size == 0:
                continue
            for kb in selected_blocks(sel_row_ptr, sel_kblk, u * nqb + qb, nkb):
                sl = np.arange(k_offsets[kb], k_offsets[kb + 1], dtype=np.int64)
                kt = sl if k_perm is None else np.asarray(k_perm, dtype=np.int64)[sl]
                if not causal:
                    tot += toks.size * kt.size
                else:
                    tot += int(np.sum(kt[None, :] <= (q_pos0 + toks)[:, None]))
        return tot

    per_unit = {}  # heads sharing a selection unit have the same count
    total = 0
    for b in range(B):
        for h in range(Hq):
            u = selection_unit(b, h, B, Hq, Hkv, sel_nb, sel_nh)
            if u not in per_unit:
                per_unit[u] = unit_pairs(u)
            total += per_unit[u]
    return total


def build_plan_w(w, fixed_tiles=False) -> Plan:
    return build_plan(w.B, w.Hq, w.Hkv, w.q_offsets, w.q_perm, w.k_offsets, w.k_perm, w.sel_nb, w.sel_nh,
                      w.sel_row_ptr, w.sel_kblk, w.causal, w.q_pos0, fixed_tiles=fixed_tiles)


# ----------------------------------------------------------------------------
# backward tables
# ----------------------------------------------------------------------------
# KPage abstract, sentence 4: the backward also walks pages that each belong to one
# K/V block, on the selected pairs only.  Readings: the key side owns its rows -- each K
# block is cut into tiles of BWD_KV_TILE slots (ceil(n/BWD_KV_TILE) per block, the last one
# short) -- and the query side is streamed in 16-row Q pages (a Q block of n slots has
# ceil(n/16) pages, as the K side in R2).  For each (unit, K block) the Q pages to visit are
# those of every Q block whose selection row holds that K block, Q blocks ascending and each
# block's pages ascending.  The dQ side owns tiles of BWD_DQ_TILE slots of each Q block and
# reuses the forward's page lists (R5).  The tile heights are a work split the page leaves
# open (it fixes only that each key row has one owner); these are the kernels' heights.
BWD_DQ_TILE = 128
BWD_KV_TILE = 64


@dataclasses.dataclass
class BwdPlan:
    qpage_qblock: np.ndarray
    qpage_slot0: np.ndarray
    qpage_nvalid: np.ndarray
    dqt_qblock: np.ndarray
    dqt_row0: np.ndarray
    dqt_rows: np.ndarray
    kvt_kblock: np.ndarray
    kvt_row0: np.ndarray
    kvt_rows: np.ndarray
    tpl_ptr: np.ndarray   # int64 [n_units * n_kblocks + 1]
    tpl_pages: np.ndarray


def build_bwd_plan(q_offsets, k_offsets, sel_nb, sel_nh, sel_row_ptr, sel_kblk) -> BwdPlan:
    nqb, nkb = len(q_offsets) - 1, len(k_offsets) - 1
    qpq, qps, qpn = [], [], []
    pages_of_qblock = []
    for qb in range(nqb):
        s0, n = int(q_offsets[qb]), int(q_offsets[qb + 1] - q_offsets[qb])
        ids = []
        for p0 in range(0, n, PAGE):
            ids.append(len(qpq))
            qpq.append(qb)
            qps.append(s0 + p0)
            qpn.append(min(PAGE, n - p0))
        pages_of_qblock.append(ids)

    def tiles(offsets, height):
        blk, row0, rows = [], [], []
        for b in range(len(offsets) - 1):
            s0, n = int(offsets[b]), int(offsets[b + 1] - offsets[b])
            for r in range(0, n, height):
                blk.append(b)
                row0.append(s0 + r)
                rows.append(min(height, n - r))
        return blk, row0, rows

    dq = tiles(q_offsets, BWD_DQ_TILE)
    kv = tiles(k_offsets, BWD_KV_TILE)
    n_units = sel_nb * sel_nh
    ptr = [0]
    pages = []
    for u in range(n_units):
        for kb in range(nkb):
            for qb in range(nqb):
                if kb in selected_blocks(sel_row_ptr, sel_kblk, u * nqb + qb, nkb):
                    pages.extend(pages_of_qblock[qb])
            ptr.append(len(pages))
    i32 = lambda a: np.asarray(a, dtype=np.int32)  # noqa: E731
    return BwdPlan(qpage_qblock=i32(qpq), qpage_slot0=i32(qps), qpage_nvalid=i32(qpn),
                   dqt_qblock=i32(dq[0]), dqt_row0=i32(dq[1]), dqt_rows=i32(dq[2]),
                   kvt_kblock=i32(kv[0]), kvt_row0=i32(kv[1]), kvt_rows=i32(kv[2]),
                   tpl_ptr=np.asarray(ptr, dtype=np.int64), tpl_pages=i32(pages))


def build_bwd_plan_w(w) -> BwdPlan:
    return build_bwd_plan(w.q_offsets, w.k_offsets, w.sel_nb, w.sel_nh, w.sel_row_ptr, w.sel_kblk)
