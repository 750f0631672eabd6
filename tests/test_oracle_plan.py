"""Pins for the oracle's plan (pages, Q-tile routing, page lists) and pair counts (CPU only).

  * a hand-worked plan (tests/golden/plan_hand.json) derived from the rules on paper;
  * closed forms for the useful pairs of the box-mask workloads (per-axis factorisation,
    tests/golden/closed_form_counts.json) and for the 1D workload (exact density);
  * explicit tile enumeration: every physical tile cell of the plan is listed, and the
    valid cells must be exactly the graph's (query, key) pairs, each once, with the
    cell count equal to the physical count;
  * structural invariants (pages owned by one block, Q tiles partition each Q block,
    query-side padding below 64 rows).
"""
import json
import os

import numpy as np
import pytest

from oracle.planner import build_plan, build_plan_w, TILE_ROWS, TILE_COLS, PAGES_PER_KTILE
from workloads.configs import make, make_random, make_cube_workload, _axis_sizes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_hand_worked_plan():
    g = _load("plan_hand.json")
    qo = np.concatenate([[0], np.cumsum(g["q_block_sizes"])]).astype(np.int32)
    ko = np.concatenate([[0], np.cumsum(g["k_block_sizes"])]).astype(np.int32)
    rp = np.concatenate([[0], np.cumsum([len(r) for r in g["selection"]])]).astype(np.int32)
    cols = np.array([c for r in g["selection"] for c in r], dtype=np.int32)
    p = build_plan(1, 1, 1, qo, None, ko, None, 1, 1, rp, cols)
    e = g["expect"]
    assert [list(x) for x in zip(p.page_kblock, p.page_slot0, p.page_nvalid)] == e["pages"]
    assert [list(x) for x in zip(p.qt_qblock, p.qt_row0, p.qt_rows, p.qt_shape)] == e["qtiles"]
    assert [p.pl_pages[p.pl_ptr[i]:p.pl_ptr[i + 1]].tolist() for i in range(len(p.pl_ptr) - 1)] == e["page_lists"]
    assert (p.physical, p.useful, p.n_ktiles) == (e["physical"], e["useful"], e["n_ktiles"])
    assert p.useful_by_shape == tuple(e["useful_by_shape"])
    assert p.physical_by_shape == tuple(e["physical_by_shape"])


def test_hand_worked_plan_causal():
    """The same hand-worked layout under a causal mask with a negative query offset: the
    useful pairs of each tile shape counted by hand; the plan itself does not change."""
    g = _load("plan_hand.json")
    c = g["causal"]
    qo = np.concatenate([[0], np.cumsum(g["q_block_sizes"])]).astype(np.int32)
    ko = np.concatenate([[0], np.cumsum(g["k_block_sizes"])]).astype(np.int32)
    rp = np.concatenate([[0], np.cumsum([len(r) for r in g["selection"]])]).astype(np.int32)
    cols = np.array([x for r in g["selection"] for x in r], dtype=np.int32)
    p = build_plan(1, 1, 1, qo, None, ko, None, 1, 1, rp, cols, causal=True, q_pos0=c["q_pos0"])
    e = g["expect"]
    assert [p.pl_pages[p.pl_ptr[i]:p.pl_ptr[i + 1]].tolist() for i in range(len(p.pl_ptr) - 1)] == e["page_lists"]
    assert p.useful == c["useful"]
    assert p.useful_by_shape == tuple(c["useful_by_shape"])
    assert p.physical_by_shape == tuple(c["physical_by_shape"])


def _axis_pairs(sizes, r):
    u = sum(sizes[i] * sizes[j] for i in range(len(sizes)) for j in range(len(sizes)) if abs(i - j) <= r)
    n = sum(1 for i in range(len(sizes)) for j in range(len(sizes)) if abs(i - j) <= r)
    return u, n


@pytest.mark.parametrize("cfg,key", [(1, "tiny3d"), (3, "videodit3d")])
def test_box_mask_counts_closed_form(cfg, key):
    g = _load("closed_form_counts.json")[key]
    per_axis = [_axis_pairs(_axis_sizes(n, c), r) for n, c, r in zip(g["grid"], g["cube"], g["radius"])]
    assert [u for u, _ in per_axis] == g["axis_useful"]
    assert [n for _, n in per_axis] == g["axis_block_pairs"]
    u_head = int(np.prod([u for u, _ in per_axis]))
    assert u_head * g["heads"] == g["useful"]
    w = make(cfg, with_tensors=False)
    assert len(w.sel_kblk) == g["block_pairs"]
    p = build_plan_w(w)
    assert p.useful == g["useful"]
    assert p.n_pages == g["pages"]
    assert p.physical == g["physical_per_head"] * g["heads"]
    if "qtiles128" in g:
        assert (p.n_qtiles128, p.n_qtiles64) == (g["qtiles128"], g["qtiles64"])
    # split by the shape of the Q tile holding the query: the routing (R4) sends a cube to
    # the 64-row shape iff it holds at most 64 tokens; with cube extents s_a(i) per axis,
    # the useful pairs of the cubes of either kind follow from the same per-axis sums
    sizes = [_axis_sizes(n, c) for n, c in zip(g["grid"], g["cube"])]
    cube_sizes = {}
    for i in range(len(sizes[0])):
        for j in range(len(sizes[1])):
            for k in range(len(sizes[2])):
                cube_sizes[(i, j, k)] = sizes[0][i] * sizes[1][j] * sizes[2][k]
    rad = g["radius"]
    split = [0, 0]
    for qc, n in cube_sizes.items():
        row = [sum(sizes[a][j] for j in range(len(sizes[a])) if abs(j - qc[a]) <= rad[a]) for a in range(3)]
        split[1 if n <= 64 else 0] += n * row[0] * row[1] * row[2]
    split = [x * g["heads"] for x in split]
    assert split == g["useful_by_shape"]
    assert p.useful_by_shape == tuple(g["useful_by_shape"])
    assert p.physical_by_shape == tuple(x * g["heads"] for x in g["physical_by_shape_per_head"])


def test_onedim_exact_density():
    g = _load("closed_form_counts.json")["onedim"]
    w = make(2, with_tensors=False)
    rows = np.diff(w.sel_row_ptr)
    assert np.all(rows == g["per_row"])
    nb = g["N"] // g["block"]
    for r in range(len(rows)):
        sel = w.sel_kblk[w.sel_row_ptr[r]:w.sel_row_ptr[r + 1]]
        assert (r % nb) in sel and len(set(sel.tolist())) == g["per_row"]
    p = build_plan_w(w)
    assert p.useful == g["useful"] == 2 ** 28
    assert p.physical == g["physical"]


def _slot_token(perm, s):
    return s if perm is None else int(perm[s])


def _graph_pairs(w, b, h):
    """(query token, key token) pairs of the graph for (b, h), by direct scanning."""
    nqb = len(w.q_offsets) - 1
    g = h // (w.Hq // w.Hkv)
    uh = h if w.sel_nh == w.Hq else (g if w.sel_nh == w.Hkv else 0)
    unit = (b if w.sel_nb == w.B else 0) * w.sel_nh + uh
    pairs = set()
    for qb in range(nqb):
        row = unit * nqb + qb
        ks = set(w.sel_kblk[w.sel_row_ptr[row]:w.sel_row_ptr[row + 1]].tolist())
        for qs in range(w.q_offsets[qb], w.q_offsets[qb + 1]):
            i = _slot_token(w.q_perm, qs)
            for kb in ks:
                for s in range(w.k_offsets[kb], w.k_offsets[kb + 1]):
                    j = _slot_token(w.k_perm, s)
                    if not w.causal or j <= w.q_pos0 + i:
                        pairs.add((i, j))
    return pairs


@pytest.mark.parametrize("kw", [
    dict(seed=61, Hq=2, Hkv=2, Nq=300, Nk=330, max_qblock=200, max_kblock=70, sel_mode="head"),
    dict(seed=62, Hq=4, Hkv=2, Nq=260, Nk=400, max_qblock=140, max_kblock=40, sel_mode="kv", use_perm=True),
    dict(seed=63, B=2, Hq=2, Hkv=1, Nq=150, Nk=500, max_qblock=150, max_kblock=64, sel_mode="batch-kv",
         causal=True, allow_empty=True),
    dict(seed=64, Hq=1, Hkv=1, Nq=333, Nk=280, max_qblock=70, max_kblock=20, sel_mode="shared",
         allow_empty=True, unsorted=True, dup=True, density=0.7),
    dict(seed=66, Hq=2, Hkv=1, Nq=280, Nk=300, max_qblock=110, max_kblock=50, sel_mode="kv", causal=True,
         use_perm=True, allow_empty=True),
])
def test_tiles_cover_graph_exactly(kw):
    w = make_random(d=8, with_tensors=False, **kw)
    p = build_plan_w(w)
    nqb = len(w.q_offsets) - 1
    cells = [0, 0]
    useful = [0, 0]
    for b in range(w.B):
        for h in range(w.Hq):
            g = h // (w.Hq // w.Hkv)
            uh = h if w.sel_nh == w.Hq else (g if w.sel_nh == w.Hkv else 0)
            unit = (b if w.sel_nb == w.B else 0) * w.sel_nh + uh
            seen = []
            for t in range(len(p.qt_qblock)):
                shape = int(p.qt_shape[t])
                assert shape == (1 if int(p.qt_rows[t]) <= 64 else 0)
                row = unit * nqb + int(p.qt_qblock[t])
                pages = p.pl_pages[p.pl_ptr[row]:p.pl_ptr[row + 1]]
                ppt = PAGES_PER_KTILE[shape]
                for k0 in range(0, len(pages), ppt):
                    tile_pages = list(pages[k0:k0 + ppt])
                    cells[shape] += TILE_ROWS[shape] * TILE_COLS[shape]
                    for r in range(int(p.qt_rows[t])):
                        i = _slot_token(w.q_perm, int(p.qt_row0[t]) + r)
                        for pg in tile_pages:
                            for c in range(int(p.page_nvalid[pg])):
                                j = _slot_token(w.k_perm, int(p.page_slot0[pg]) + c)
                                if not w.causal or j <= w.q_pos0 + i:
                                    seen.append((i, j))
                                    useful[shape] += 1
            assert len(seen) == len(set(seen)), "a pair is covered twice"
            assert set(seen) == _graph_pairs(w, b, h)
    assert sum(cells) == p.physical
    assert sum(useful) == p.useful
    # the split by the shape of the tile that holds the query, cell by cell
    assert tuple(cells) == p.physical_by_shape
    assert tuple(useful) == p.useful_by_shape
    assert p.n_ktiles * 16384 == p.physical


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_structural_invariants(cfg):
    w = make(cfg, with_tensors=False)
    p = build_plan_w(w)
    # pages: owned by one block, 16 rows except a block's last page
    for kb in range(w.n_kblocks):
        idx = np.nonzero(p.page_kblock == kb)[0]
        n = int(w.k_offsets[kb + 1] - w.k_offsets[kb])
        assert int(p.page_nvalid[idx].sum()) == n
        assert np.all(p.page_nvalid[idx[:-1]] == 16) if idx.size else n == 0
        assert np.all(p.page_slot0[idx] >= w.k_offsets[kb])
        assert np.all(p.page_slot0[idx] + p.page_nvalid[idx] <= w.k_offsets[kb + 1])
    # Q tiles partition each block, padding below 64 rows
    for qb in range(w.n_qblocks):
        idx = np.nonzero(p.qt_qblock == qb)[0]
        n = int(w.q_offsets[qb + 1] - w.q_offsets[qb])
        assert int(p.qt_rows[idx].sum()) == n
        cap = sum(TILE_ROWS[int(s)] for s in p.qt_shape[idx])
        assert 0 <= cap - n < 64
        assert np.array_equal(p.qt_row0[idx], w.q_offsets[qb] + np.concatenate([[0], np.cumsum(p.qt_rows[idx])[:-1]]))
    assert p.physical >= p.useful


def test_cube_physical_independent_derivation():
    """Video-DiT cube workload: physical pairs per head from cube geometry alone."""
    w = make_cube_workload("c3", 3, (21, 45, 80), (2, 8, 8), (1, 2, 2), B=1, H=1, d=128, with_tensors=False)
    st, sh, sw = _axis_sizes(21, 2), _axis_sizes(45, 8), _axis_sizes(80, 8)
    cubes = [(a, b, c) for a in range(len(st)) for b in range(len(sh)) for c in range(len(sw))]
    size = {x: st[x[0]] * sh[x[1]] * sw[x[2]] for x in cubes}
    phys = {128: 0, 256: 0}
    for qc in cubes:
        pages = sum(-(-size[kc] // 16) for kc in cubes
                    if abs(kc[0] - qc[0]) <= 1 and abs(kc[1] - qc[1]) <= 2 and abs(kc[2] - qc[2]) <= 2)
        n = size[qc]
        tiles = [128] * (n // 128) + ([64] if 0 < n % 128 <= 64 else [128] if n % 128 else [])
        for rows in tiles:
            width = 128 if rows == 128 else 256
            phys[width] += rows * width * -(-pages // (width // 16))
    p = build_plan_w(w)
    assert phys[128] + phys[256] == p.physical == 485621760
    # split by tile width: 128-key tiles belong to the 128-row shape, 256-key tiles to the 64-row one
    assert (phys[128], phys[256]) == p.physical_by_shape == (472940544, 12681216)


# ---------------------------------------------------------------------------
# backward tables
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [61, 62, 63, 64])
def test_bwd_lists_enumerate_graph_transpose(seed):
    """Brute force over (unit, query slot, key block): the Q page list of (unit, K block)
    covers exactly the query slots whose Q block selects that K block, each once, in slot
    order; its pages never straddle Q blocks; the owned tiles of each side (128 slots on the
    Q side, 64 on the K side) partition every block in order."""
    from oracle.planner import build_bwd_plan_w
    w = make_random(seed, B=2, Hq=4, Hkv=2, Nq=300, Nk=260, d=64, max_qblock=70, max_kblock=50, density=0.35,
                    sel_mode="batch-kv", allow_empty=True, unsorted=True, dup=True, with_tensors=False)
    bp = build_bwd_plan_w(w)
    nqb, nkb = w.n_qblocks, w.n_kblocks
    qblk_of_slot = np.repeat(np.arange(nqb), np.diff(w.q_offsets))
    for u in range(w.sel_nb * w.sel_nh):
        for kb in range(nkb):
            row = u * nkb + kb
            pages = bp.tpl_pages[bp.tpl_ptr[row]:bp.tpl_ptr[row + 1]]
            slots = []
            for pg in pages:
                s0, nv = int(bp.qpage_slot0[pg]), int(bp.qpage_nvalid[pg])
                assert 1 <= nv <= 16
                assert np.all(qblk_of_slot[s0:s0 + nv] == bp.qpage_qblock[pg])
                slots.extend(range(s0, s0 + nv))
            want = [s for s in range(w.Nq)
                    if kb in set(w.sel_kblk[w.sel_row_ptr[u * nqb + qblk_of_slot[s]]:
                                            w.sel_row_ptr[u * nqb + qblk_of_slot[s] + 1]].tolist())]
            assert slots == want, (u, kb)
    for offs, blk, row0, rows, height in ((w.q_offsets, bp.dqt_qblock, bp.dqt_row0, bp.dqt_rows, 128),
                                          (w.k_offsets, bp.kvt_kblock, bp.kvt_row0, bp.kvt_rows, 64)):
        covered = []
        for b, r0, n in zip(blk, row0, rows):
            assert 1 <= n <= height and offs[b] <= r0 and r0 + n <= offs[b + 1]
            # a block's tiles are full except its last
            assert n == height or r0 + n == offs[b + 1]
            covered.extend(range(r0, r0 + n))
        assert covered == list(range(int(offs[-1])))


@pytest.mark.parametrize("cfg", [1, 3])
def test_bwd_lists_count_the_forward_useful_pairs(cfg):
    """Non-causal, one unit: sum over K blocks of (keys in the block) x (query rows of its
    Q page list) = the forward plan's useful pairs per head (closed form in the golden file)."""
    from oracle.planner import build_bwd_plan_w
    w = make(cfg, with_tensors=False)
    bp = build_bwd_plan_w(w)
    per_head = 0
    for kb in range(w.n_kblocks):
        pages = bp.tpl_pages[bp.tpl_ptr[kb]:bp.tpl_ptr[kb + 1]]
        per_head += int(w.k_offsets[kb + 1] - w.k_offsets[kb]) * int(bp.qpage_nvalid[pages].sum())
    g = _load("closed_form_counts.json")
    key = {1: "tiny3d", 3: "videodit3d"}[cfg]
    assert per_head * w.Hq == g[key]["useful"]


@pytest.mark.parametrize("cfg,key", [(1, "tiny3d"), (3, "videodit3d")])
def test_fixed_tiles_closed_form(cfg, key):
    """Fixed-tile baseline on blocks of at most 128 tokens: one 128x128 tile per (Q block,
    selected K block) pair, so physical = 16384 x block pairs x heads (block pairs from the
    per-axis closed form); the useful pairs are those of the packed plan."""
    g = _load("closed_form_counts.json")[key]
    w = make(cfg, with_tensors=False)
    fx = build_plan_w(w, fixed_tiles=True)
    assert fx.physical == 128 * 128 * g["block_pairs"] * g["heads"]
    assert fx.useful == g["useful"]
    assert fx.n_qtiles64 == 0
    ratio = fx.physical / fx.useful
    assert abs(ratio - {1: 9.4815, 3: 1.1620}[cfg]) < 1e-4
