"""Seeded generators for the five benchmark workloads and for small fuzz cases.

Every generator returns a :class:`Workload` holding
  * the problem shape (B, Hq, Hkv, Nq, Nk, d), softmax scale, causal flag and
    the absolute position of query 0;
  * one token layout per side: ``offsets`` (n_blocks + 1 slot boundaries) and an
    optional ``perm`` (slot -> token index, ``None`` = identity);
  * a block selection in CSR form over (unit, Q block) rows, where a unit is a
    (batch, head) group: ``sel_nb`` is 1 or B, ``sel_nh`` is 1, Hkv or Hq;
  * Q [B, Nq, Hq, d], K and V [B, Nk, Hkv, d] as bf16 bit patterns (uint16).

Random draws use ``numpy.random.default_rng(seed)`` (PCG64) in a fixed order:
structure first (masks, partitions, selections), then Q, K, V, each drawn as
float32 N(0, 1) over the whole tensor in C order and rounded to bf16 with
round-to-nearest-even.  The only data-dependent structure is the chunk
selection of the long-context GQA workload, which is derived from the drawn Q
and K after they exist (chunk summaries, CISA abstract sentences 3-5) by a
selection function the caller passes in: this module holds no arithmetic of the
method itself.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

CONFIG_NAMES = {
    1: "tiny-3d-5x12x12-cubes2x4x8-d64",
    2: "1d-8192-blocks128-density25-h16-d128",
    3: "videodit-3d-21x45x80-cubes2x8x8-h40-d128",
    4: "indep-qk-partitions-75600-h40-d128",
    5: "chunk-gqa-prefill-b4-h64kv8-262144-d128",
}

_CHUNK = 1 << 24  # elements per random draw chunk (bounded host memory)


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    q_offsets: np.ndarray
    q_perm: Optional[np.ndarray]
    k_offsets: np.ndarray
    k_perm: Optional[np.ndarray]
    sel_nb: int
    sel_nh: int
    sel_row_ptr: np.ndarray
    sel_kblk: np.ndarray
    causal: bool = False
    q_pos0: int = 0
    scale: float = 0.0
    q: Optional[np.ndarray] = None
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    do: Optional[np.ndarray] = None  # upstream gradient of O (backward only), drawn on demand
    # dispatch order of the Q blocks (a locality hint for the kernels; None = ascending)
    q_block_order: Optional[np.ndarray] = None
    rng: Optional[np.random.Generator] = dataclasses.field(default=None, repr=False)

    @property
    def n_qblocks(self) -> int:
        return int(self.q_offsets.shape[0] - 1)

    @property
    def n_kblocks(self) -> int:
        return int(self.k_offsets.shape[0] - 1)


# ----------------------------------------------------------------------------
# bf16 encoding of generated values (input preparation only)
# ----------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape: Sequence[int]) -> np.ndarray:
    """Draw float32 N(0,1) over ``shape`` in C order (in bounded chunks) and round to bf16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    pos = 0
    while pos < n:
        m = min(_CHUNK, n - pos)
        out[pos:pos + m] = bf16_bits_from_f32(rng.standard_normal(m, dtype=np.float32))
        pos += m
    return out.reshape(tuple(shape))


# ----------------------------------------------------------------------------
# layouts and selections
# ----------------------------------------------------------------------------
def _axis_sizes(n: int, c: int) -> List[int]:
    """Cube extents along one axis: full cubes from the origin, a partial one at the high end."""
    s = [c] * (n // c)
    if n % c:
        s.append(n % c)
    return s


def cube_layout(grid: Tuple[int, int, int], cube: Tuple[int, int, int]):
    """Token grid (T, H, W) cut into cubes anchored at the origin.

    Tokens are flattened in cube order: cubes in raster order over their (t, h, w)
    cube coordinates (t slowest), tokens inside a cube in raster order.  Each cube is
    therefore a contiguous slot range and the slot->token permutation is the
    identity.  Returns (offsets int32[n+1], coords int32[n, 3]).
    """
    st, sh, sw = (_axis_sizes(g, c) for g, c in zip(grid, cube))
    sizes, coords = [], []
    for it, a in enumerate(st):
        for ih, b in enumerate(sh):
            for iw, c in enumerate(sw):
                sizes.append(a * b * c)
                coords.append((it, ih, iw))
    offs = np.zeros(len(sizes) + 1, dtype=np.int64)
    offs[1:] = np.cumsum(sizes)
    return offs.astype(np.int32), np.asarray(coords, dtype=np.int32)


def cube_dispatch_order(coords: np.ndarray, slab: int = 2) -> np.ndarray:
    """Cubes ordered in slabs of ``slab`` cube columns along w; inside a slab by t, then h,
    then w.  The Q tiles that run together on one XCD are then the cubes of one or two t
    planes of a narrow w slab: their page lists cover nearly the same K blocks in the same
    order, so the pages one tile loads are still in that XCD's L2 when its neighbours reach
    them.  On the video-DiT grid an LRU model of one XCD's L2 gives 28% misses in raster
    (t, h, w) order, 18% in (h, t, w) order and 9% with slabs of two; the launch measured
    9.97, 9.85 and 9.71 ms in those orders (alternating runs on one MI355X)."""
    c = np.asarray(coords)
    return np.lexsort((c[:, 2] % slab, c[:, 1], c[:, 0], c[:, 2] // slab)).astype(np.int32)


def box_selection(coords: np.ndarray, radius: Tuple[int, int, int]):
    """Q cube i selects K cube j iff |ci - cj| <= radius on every axis (same cube grid on both sides)."""
    r = np.asarray(radius, dtype=np.int32)
    row_ptr = [0]
    cols: List[int] = []
    for i in range(coords.shape[0]):
        ok = np.all(np.abs(coords - coords[i]) <= r, axis=1)
        js = np.nonzero(ok)[0]
        cols.extend(int(j) for j in js)
        row_ptr.append(len(cols))
    return np.asarray(row_ptr, dtype=np.int32), np.asarray(cols, dtype=np.int32)


def uniform_layout(n: int, block: int) -> np.ndarray:
    nb = (n + block - 1) // block
    offs = np.minimum(np.arange(nb + 1, dtype=np.int64) * block, n)
    return offs.astype(np.int32)


def random_partition(rng: np.random.Generator, n: int, lo: int, hi: int):
    """Random clusters: a permutation of the n tokens cut into runs of lo..hi tokens.

    Sizes are drawn one at a time from integers in [lo, hi] until they cover n; the
    last is truncated, and merged into the previous cluster when it falls below lo.
    Returns (offsets int32, perm int32 slot->token).
    """
    perm = rng.permutation(n).astype(np.int32)
    sizes: List[int] = []
    total = 0
    while total < n:
        s = int(rng.integers(lo, hi + 1))
        s = min(s, n - total)
        sizes.append(s)
        total += s
    if len(sizes) > 1 and sizes[-1] < lo:
        last = sizes.pop()
        sizes[-1] += last
    offs = np.zeros(len(sizes) + 1, dtype=np.int64)
    offs[1:] = np.cumsum(sizes)
    return offs.astype(np.int32), perm


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------
def _tensors(w: Workload, rng: np.random.Generator) -> None:
    w.q = normal_bf16(rng, (w.B, w.Nq, w.Hq, w.d))
    w.k = normal_bf16(rng, (w.B, w.Nk, w.Hkv, w.d))
    w.v = normal_bf16(rng, (w.B, w.Nk, w.Hkv, w.d))
    w.rng = rng  # dO, when a backward needs it, continues this stream


def draw_dout(w: Workload) -> np.ndarray:
    """The upstream gradient dO ~ N(0,1) in bf16, shaped like O, drawn once from the
    workload's generator right after Q, K and V."""
    if w.do is None:
        if w.rng is None:
            raise ValueError("the workload has no tensors")
        w.do = normal_bf16(w.rng, (w.B, w.Nq, w.Hq, w.d))
    return w.do


def make_cube_workload(name, seed, grid, cube, radius, B, H, d, with_tensors=True) -> Workload:
    rng = np.random.default_rng(seed)
    offs, coords = cube_layout(grid, cube)
    rp, cols = box_selection(coords, radius)
    n = int(offs[-1])
    w = Workload(name=name, seed=seed, B=B, Hq=H, Hkv=H, Nq=n, Nk=n, d=d,
                 q_offsets=offs, q_perm=None, k_offsets=offs.copy(), k_perm=None,
                 sel_nb=1, sel_nh=1, sel_row_ptr=rp, sel_kblk=cols, scale=1.0 / np.sqrt(d),
                 q_block_order=cube_dispatch_order(coords))
    if with_tensors:
        _tensors(w, rng)
    return w


def make_1d_random(name, seed, N, block, H, d, per_row, B=1, with_tensors=True) -> Workload:
    """Per-(head, Q-block) random block mask: the diagonal block plus ``per_row - 1``
    others drawn uniformly without replacement (exact density per_row / n_blocks)."""
    rng = np.random.default_rng(seed)
    offs = uniform_layout(N, block)
    nb = offs.shape[0] - 1
    rp = [0]
    cols: List[int] = []
    for _h in range(H):
        for qb in range(nb):
            others = np.array([j for j in range(nb) if j != qb], dtype=np.int64)
            pick = rng.choice(nb - 1, size=per_row - 1, replace=False)
            row = sorted([qb] + [int(others[p]) for p in pick])
            cols.extend(row)
            rp.append(len(cols))
    w = Workload(name=name, seed=seed, B=B, Hq=H, Hkv=H, Nq=N, Nk=N, d=d,
                 q_offsets=offs, q_perm=None, k_offsets=offs.copy(), k_perm=None,
                 sel_nb=1, sel_nh=H, sel_row_ptr=np.asarray(rp, np.int32),
                 sel_kblk=np.asarray(cols, np.int32), scale=1.0 / np.sqrt(d))
    if with_tensors:
        _tensors(w, rng)
    return w


def make_partitions(name, seed, N, H, d, lo=16, hi=300, key_frac=0.15, B=1, with_tensors=True) -> Workload:
    """Independent random Q and K clusterings; each Q cluster greedily takes K clusters
    in a random order while the running key count stays within floor(key_frac * N)."""
    rng = np.random.default_rng(seed)
    qoffs, qperm = random_partition(rng, N, lo, hi)
    koffs, kperm = random_partition(rng, N, lo, hi)
    ksz = np.diff(koffs.astype(np.int64))
    budget = int(np.floor(key_frac * N))
    rp = [0]
    cols: List[int] = []
    for _qc in range(qoffs.shape[0] - 1):
        order = rng.permutation(ksz.shape[0])
        tot = 0
        chosen = []
        for kc in order:
            if tot + int(ksz[kc]) > budget:
                break
            tot += int(ksz[kc])
            chosen.append(int(kc))
        cols.extend(sorted(chosen))
        rp.append(len(cols))
    w = Workload(name=name, seed=seed, B=B, Hq=H, Hkv=H, Nq=N, Nk=N, d=d,
                 q_offsets=qoffs, q_perm=qperm, k_offsets=koffs, k_perm=kperm,
                 sel_nb=1, sel_nh=1, sel_row_ptr=np.asarray(rp, np.int32),
                 sel_kblk=np.asarray(cols, np.int32), scale=1.0 / np.sqrt(d))
    if with_tensors:
        _tensors(w, rng)
    return w


def make_chunk_gqa(name, seed, B, Hq, Hkv, d, Nk, Nq, chunk, topk, *, chunk_select, causal=True,
                   with_tensors=True) -> Workload:
    """Long-context GQA prefill over selected KV chunks.  The queries are the last Nq
    positions of an Nk-token sequence (query i sits at absolute position Nk - Nq + i);
    one Q block holds all of them (QShare) and each (batch, KV group) unit selects the
    same chunk set for all its query heads.

    The selection is computed from the drawn Q and K by ``chunk_select(w, chunk, topk)``,
    which returns int32 [B * Hkv, topk] (ascending chunk ids per (batch, KV group)).  The
    chunk scoring is part of the method (CISA abstract, sentences 3-5), so this module only
    draws the inputs and the caller brings the selection: the tests use the float64 oracle's,
    the benchmark the GPU's (which the tests check against the oracle)."""
    rng = np.random.default_rng(seed)
    qoffs = np.array([0, Nq], dtype=np.int32)
    koffs = uniform_layout(Nk, chunk)
    w = Workload(name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d,
                 q_offsets=qoffs, q_perm=None, k_offsets=koffs, k_perm=None,
                 sel_nb=B, sel_nh=Hkv, sel_row_ptr=np.zeros(1, np.int32), sel_kblk=np.zeros(0, np.int32),
                 causal=causal, q_pos0=Nk - Nq, scale=1.0 / np.sqrt(d))
    if not with_tensors:
        raise ValueError("the chunk selection is derived from Q and K; tensors are required")
    _tensors(w, rng)
    sel = np.asarray(chunk_select(w, chunk, topk), dtype=np.int32)
    if sel.shape != (B * Hkv, topk):
        raise ValueError(f"chunk_select returned shape {sel.shape}, expected {(B * Hkv, topk)}")
    w.sel_row_ptr = (np.arange(B * Hkv + 1, dtype=np.int64) * topk).astype(np.int32)
    w.sel_kblk = sel.reshape(-1)
    return w


def make(cfg: int, seed: Optional[int] = None, with_tensors: bool = True, chunk_select=None) -> Workload:
    """The five benchmark workloads at full size; seed defaults to the config number.
    Workload 5 needs ``chunk_select`` (see make_chunk_gqa)."""
    s = cfg if seed is None else seed
    name = CONFIG_NAMES[cfg]
    if cfg == 1:
        return make_cube_workload(name, s, (5, 12, 12), (2, 4, 8), (1, 1, 1), B=1, H=2, d=64, with_tensors=with_tensors)
    if cfg == 2:
        return make_1d_random(name, s, N=8192, block=128, H=16, d=128, per_row=16, with_tensors=with_tensors)
    if cfg == 3:
        return make_cube_workload(name, s, (21, 45, 80), (2, 8, 8), (1, 2, 2), B=1, H=40, d=128, with_tensors=with_tensors)
    if cfg == 4:
        return make_partitions(name, s, N=75600, H=40, d=128, with_tensors=with_tensors)
    if cfg == 5:
        if chunk_select is None:
            raise ValueError("workload 5 selects its chunks from Q and K: pass chunk_select")
        return make_chunk_gqa(name, s, B=4, Hq=64, Hkv=8, d=128, Nk=262144, Nq=2048, chunk=64, topk=2048,
                              chunk_select=chunk_select, with_tensors=with_tensors)
    raise ValueError(f"unknown config {cfg}")


# ----------------------------------------------------------------------------
# small random cases for parity and fuzzing
# ----------------------------------------------------------------------------
def random_layout(rng: np.random.Generator, n: int, max_block: int, allow_empty: bool, use_perm: bool):
    sizes: List[int] = []
    tot = 0
    while tot < n:
        lo = 0 if allow_empty else 1
        s = int(rng.integers(lo, max_block + 1))
        s = min(s, n - tot)
        sizes.append(s)
        tot += s
    offs = np.zeros(len(sizes) + 1, dtype=np.int64)
    offs[1:] = np.cumsum(sizes)
    perm = rng.permutation(n).astype(np.int32) if use_perm else None
    return offs.astype(np.int32), perm


def make_random(seed: int, B=1, Hq=2, Hkv=2, Nq=300, Nk=300, d=64, max_qblock=200, max_kblock=200,
                density=0.5, sel_mode="head", allow_empty=False, use_perm=False, causal=False,
                q_pos0=None, with_tensors=True, unsorted=False, dup=False) -> Workload:
    """Random layouts and selections for parity tests.  ``sel_mode``: 'shared' (one unit),
    'kv' (per KV head), 'head' (per query head), 'batch-kv' (per batch and KV head)."""
    rng = np.random.default_rng(seed)
    qoffs, qperm = random_layout(rng, Nq, max_qblock, allow_empty, use_perm)
    koffs, kperm = random_layout(rng, Nk, max_kblock, allow_empty, use_perm)
    nqb, nkb = qoffs.shape[0] - 1, koffs.shape[0] - 1
    nb = B if sel_mode == "batch-kv" else 1
    nh = {"shared": 1, "kv": Hkv, "head": Hq, "batch-kv": Hkv}[sel_mode]
    rp = [0]
    cols: List[int] = []
    for _u in range(nb * nh):
        for _qb in range(nqb):
            m = rng.random(nkb) < density
            row = [int(j) for j in np.nonzero(m)[0]]
            if unsorted:
                row = [row[i] for i in rng.permutation(len(row))]
            if dup and row:
                row = row + [row[int(rng.integers(0, len(row)))]]
            cols.extend(row)
            rp.append(len(cols))
    w = Workload(name=f"random-{seed}", seed=seed, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d,
                 q_offsets=qoffs, q_perm=qperm, k_offsets=koffs, k_perm=kperm,
                 sel_nb=nb, sel_nh=nh, sel_row_ptr=np.asarray(rp, np.int32),
                 sel_kblk=np.asarray(cols, np.int32), causal=causal,
                 q_pos0=(Nk - Nq if q_pos0 is None else q_pos0) if causal else 0,
                 scale=1.0 / np.sqrt(d))
    if with_tensors:
        _tensors(w, rng)
    return w
