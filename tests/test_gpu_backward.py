"""GPU parity of libbsattn's backward pass against the float64 oracle (needs an MI355X).

Every call goes through the C ABI (``bsattn_fwd`` for O and LSE, then ``bsattn_bwd``) via
the ctypes binding; gradients are NaN-poisoned before each launch so unwritten rows show
up.  The oracle's gradients use its own exact O and LSE; the GPU path uses the forward's
bf16 O and fp32 LSE, as a training step would.

Bar, per gradient tensor G against the oracle R (a derived tolerance: the forward's bar
states none for gradients).  P^ and dS enter the MFMAs as bf16 (relative rounding 2^-9 on
each term of sums whose terms have random signs) and the outputs are stored as bf16
(2^-9 relative), so the error of an entry is a few 2^-9 of the tensor's scale:
    max |G - R|  <= 2e-2 * max |R|      mean |G - R| <= 1e-2 * mean |R|
Entries whose reference is exactly zero stay within 1e-5 * max |R| (rounding: a query with
a single key has dS = 0 exactly, which the GPU's differently ordered fp32 sums give to about
1e-8); the backward's own structural zeros -- keys that no query reaches and queries without
keys -- are checked to be exactly zero.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_fwd_amd as bs
from oracle.attention import masked_attention_bwd_w, masked_attention_w
from workloads.configs import make, make_random, make_partitions, draw_dout
from tests.oracle_select import oracle_chunk_select

pytestmark = pytest.mark.gpu

G_MAX, G_MEAN = 2e-2, 1e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_gpu_bwd(w, plan=None, poison=True):
    if plan is None:
        plan = bs.Plan.from_workload(w).upload()
    q, k, v, do = _dev(w.q), _dev(w.k), _dev(w.v), _dev(draw_dout(w))
    o, lse = plan.fwd(q, k, v, scale=w.scale)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if poison:
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
    plan.bwd(q, k, v, o, lse, do, dq, dk, dv, scale=w.scale)
    torch.cuda.synchronize()
    return _np(dq), _np(dk), _np(dv), plan


def check_grad(g, r, label):
    assert np.all(np.isfinite(g)), f"{label}: non-finite gradient (unwritten rows?)"
    zero = r == 0.0
    scale_max = np.abs(r).max()
    if scale_max == 0.0:
        assert not g.any(), f"{label}: nonzero gradient where every reference entry is zero"
        return
    assert np.abs(g[zero]).max(initial=0.0) <= 1e-5 * scale_max, f"{label}: nonzero where the reference is zero"
    err = np.abs(g - r)
    rel_max = err.max() / scale_max
    rel_mean = err.mean() / np.abs(r).mean()
    _say(f"{label}: max {err.max():.3e} ({rel_max:.2e} of max|ref| {scale_max:.3e}), "
         f"mean {err.mean():.3e} ({rel_mean:.2e} of mean|ref|)")
    assert rel_max <= G_MAX, f"{label}: max error {rel_max:.3e} of the tensor's max"
    assert rel_mean <= G_MEAN, f"{label}: mean error {rel_mean:.3e} of the tensor's mean"


def structural_zeros(w, dq, dk, dv):
    """Queries with no key (oracle LSE = -inf) get dQ = 0 and keys that no query of a head
    group reaches get dK = dV = 0, exactly."""
    _, L = masked_attention_w(w)
    grp = w.Hq // w.Hkv
    for b in range(w.B):
        for h in range(w.Hq):
            dead = ~np.isfinite(L[b, h])
            assert not dq[b, dead, h].any(), f"dQ of queries without keys (b{b} h{h})"
    # a key is reached iff some query head of its group has a query whose row holds it
    reached = np.zeros((w.B, w.Nk, w.Hkv), dtype=bool)
    ktok_blk = np.zeros(w.Nk, np.int64)
    for kb in range(w.n_kblocks):
        sl = np.arange(w.k_offsets[kb], w.k_offsets[kb + 1])
        ktok_blk[sl if w.k_perm is None else w.k_perm[sl]] = kb
    qtok_blk = np.zeros(w.Nq, np.int64)
    for qb in range(w.n_qblocks):
        sl = np.arange(w.q_offsets[qb], w.q_offsets[qb + 1])
        qtok_blk[sl if w.q_perm is None else w.q_perm[sl]] = qb
    for b in range(w.B):
        for h in range(w.Hq):
            ub = b if w.sel_nb == w.B else 0
            uh = h if w.sel_nh == w.Hq else (h // grp if w.sel_nh == w.Hkv else 0)
            unit = ub * w.sel_nh + uh
            for qb in range(w.n_qblocks):
                members = np.nonzero(qtok_blk == qb)[0]
                if members.size == 0:
                    continue
                sel = w.sel_kblk[w.sel_row_ptr[unit * w.n_qblocks + qb]:w.sel_row_ptr[unit * w.n_qblocks + qb + 1]]
                keys = np.nonzero(np.isin(ktok_blk, sel))[0]
                if w.causal:
                    keys = keys[keys <= w.q_pos0 + members.max()]
                reached[b, keys, h // grp] = True
    assert not dk[~reached].any() and not dv[~reached].any(), "dK/dV of keys that no query reaches"


def check_full(w, label):
    _say(f"[gpu-bwd] {label}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d} causal={w.causal}")
    dq, dk, dv, _ = run_gpu_bwd(w)
    structural_zeros(w, dq, dk, dv)
    rq, rk, rv = masked_attention_bwd_w(w, draw_dout(w))
    check_grad(dq, rq, f"{label} dQ")
    check_grad(dk, rk, f"{label} dK")
    check_grad(dv, rv, f"{label} dV")


# ---------------------------------------------------------------------------
# small cases: every gradient entry compared
# ---------------------------------------------------------------------------
BWD_CASES = [
    dict(seed=201, B=1, Hq=2, Hkv=2, Nq=700, Nk=900, d=128, max_qblock=300, max_kblock=100, sel_mode="head"),
    dict(seed=202, B=1, Hq=2, Hkv=2, Nq=650, Nk=800, d=64, max_qblock=260, max_kblock=70, sel_mode="kv"),
    dict(seed=203, B=2, Hq=4, Hkv=2, Nq=500, Nk=700, d=128, max_qblock=200, max_kblock=64, sel_mode="batch-kv",
         use_perm=True),
    dict(seed=204, B=1, Hq=4, Hkv=1, Nq=400, Nk=1100, d=128, max_qblock=400, max_kblock=64, sel_mode="shared",
         causal=True),
    dict(seed=205, B=1, Hq=2, Hkv=2, Nq=450, Nk=450, d=64, max_qblock=100, max_kblock=40, sel_mode="head",
         causal=True, use_perm=True, allow_empty=True, density=0.3),
    dict(seed=206, B=1, Hq=4, Hkv=2, Nq=333, Nk=517, d=128, max_qblock=64, max_kblock=17, sel_mode="head",
         allow_empty=True, density=0.1, unsorted=True, dup=True),
    dict(seed=207, B=1, Hq=1, Hkv=1, Nq=129, Nk=257, d=128, max_qblock=129, max_kblock=257, sel_mode="shared",
         density=1.0),
    dict(seed=208, B=1, Hq=2, Hkv=2, Nq=64, Nk=16, d=64, max_qblock=64, max_kblock=16, sel_mode="head",
         density=1.0),
    # dQ tiles of both kinds (more than 64 rows, and 1..64 rows with the key split) with
    # permuted keys under a causal mask at head dim 128
    dict(seed=209, B=1, Hq=2, Hkv=1, Nq=620, Nk=580, d=128, max_qblock=90, max_kblock=45, sel_mode="kv",
         causal=True, use_perm=True, allow_empty=True, density=0.35),
    # only split dQ tiles (blocks of 1..64 rows), causal with identity layouts, head dim 64
    dict(seed=210, B=1, Hq=2, Hkv=2, Nq=700, Nk=500, d=64, max_qblock=64, max_kblock=50, sel_mode="head",
         causal=True, q_pos0=-40, density=0.4),
]


@pytest.mark.parametrize("kw", BWD_CASES, ids=[f"seed{c['seed']}" for c in BWD_CASES])
def test_bwd_random_full(kw):
    check_full(make_random(**kw), f"random-{kw['seed']}")


def test_bwd_tiny_3d_full():
    check_full(make(1), "tiny-3d")


def test_bwd_empty_selection_gives_zeros():
    w = make_random(211, B=1, Hq=2, Hkv=2, Nq=200, Nk=300, d=128, max_qblock=90, max_kblock=50, sel_mode="head")
    w.sel_row_ptr = np.zeros_like(w.sel_row_ptr)
    w.sel_kblk = np.zeros(0, np.int32)
    dq, dk, dv, _ = run_gpu_bwd(w)
    assert not dq.any() and not dk.any() and not dv.any()


def test_bwd_deterministic_bitwise():
    w = make_random(212, B=1, Hq=4, Hkv=2, Nq=600, Nk=600, d=128, max_qblock=150, max_kblock=60, sel_mode="head",
                    use_perm=True)
    a = run_gpu_bwd(w)
    b = run_gpu_bwd(w, plan=a[3])
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)


def test_bwd_partitions_scaled_full():
    # the independent Q/K partition workload's structure at 6,000 tokens and 2 heads
    w = make_partitions("partitions-scaled", 4, N=6000, H=2, d=128)
    check_full(w, "partitions-6000")


def test_bwd_partitions_full_size_sampled():
    # independent Q/K partitions at full size (75,600 tokens, 40 heads): dQ of sampled queries
    # and dK/dV of every key of one K cluster, in one head, against the oracle
    w = make(4)
    _say(f"[gpu-bwd] partitions full size: Nq={w.Nq} Hq={w.Hq} d={w.d}")
    dq, dk, dv, plan = run_gpu_bwd(w)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
    rng = np.random.default_rng(4)
    h = 17
    qtoks = np.sort(rng.choice(w.Nq, 48, replace=False))
    kb = int(rng.integers(0, w.n_kblocks))
    sl = np.arange(w.k_offsets[kb], w.k_offsets[kb + 1])
    ktoks = np.sort(w.k_perm[sl] if w.k_perm is not None else sl)
    _say(f"[gpu-bwd] oracle: {len(qtoks)} query rows and K cluster {kb} ({len(ktoks)} keys) of head {h}")
    (rq,), ((rk, rv),) = masked_attention_bwd_w(w, draw_dout(w), q_rows=[(0, h, qtoks)], k_rows=[(0, h, ktoks)])
    check_grad(dq[0, qtoks, h], rq, "partitions dQ rows")
    check_grad(dk[0, ktoks, h], rk, "partitions dK cluster")
    check_grad(dv[0, ktoks, h], rv, "partitions dV cluster")


def test_bwd_videodit_full_size_sampled():
    # video-DiT 3D at full size (75,600 tokens, 40 heads, cube layout): dQ of sampled queries
    # and dK/dV of every key of one cube, in one head, against the oracle
    w = make(3)
    _say(f"[gpu-bwd] video-DiT full size: Nq={w.Nq} Hq={w.Hq} d={w.d}")
    dq, dk, dv, plan = run_gpu_bwd(w)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
    rng = np.random.default_rng(3)
    h = 29
    qtoks = np.sort(rng.choice(w.Nq, 48, replace=False))
    kb = int(rng.integers(0, w.n_kblocks))
    ktoks = np.arange(w.k_offsets[kb], w.k_offsets[kb + 1])
    _say(f"[gpu-bwd] oracle: {len(qtoks)} query rows and cube {kb} ({len(ktoks)} keys) of head {h}")
    (rq,), ((rk, rv),) = masked_attention_bwd_w(w, draw_dout(w), q_rows=[(0, h, qtoks)], k_rows=[(0, h, ktoks)])
    check_grad(dq[0, qtoks, h], rq, "video-DiT dQ rows")
    check_grad(dk[0, ktoks, h], rk, "video-DiT dK cube")
    check_grad(dv[0, ktoks, h], rv, "video-DiT dV cube")


def test_bwd_chunk_gqa_full_size_sampled():
    # chunk-indexed GQA prefill at full size (4 x 262,144 keys, 64 query heads in 8 KV groups,
    # causal): dQ of sampled query rows against the oracle (each reaches its group's 131,072
    # selected keys), and exact zeros in dK/dV for chunks that a group does not select
    w = make(5, chunk_select=oracle_chunk_select)
    _say(f"[gpu-bwd] chunk GQA full size: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} causal={w.causal}")
    dq, dk, dv, plan = run_gpu_bwd(w)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
    rng = np.random.default_rng(5)
    b, h = 2, 45
    qtoks = np.sort(rng.choice(w.Nq, 12, replace=False))
    _say(f"[gpu-bwd] oracle: {len(qtoks)} query rows of (batch {b}, head {h})")
    (rq,), _ = masked_attention_bwd_w(w, draw_dout(w), q_rows=[(b, h, qtoks)])
    check_grad(dq[b, qtoks, h], rq, "chunk GQA dQ rows")
    g = h // (w.Hq // w.Hkv)
    assert w.n_qblocks == 1 and w.sel_nb == w.B and w.sel_nh == w.Hkv  # one query block, a selection per (b, g)
    unit = b * w.sel_nh + g
    selected = set(int(c) for c in w.sel_kblk[w.sel_row_ptr[unit]:w.sel_row_ptr[unit + 1]])
    unselected = [c for c in range(w.n_kblocks) if c not in selected][:64]
    for c in unselected:
        sl = slice(int(w.k_offsets[c]), int(w.k_offsets[c + 1]))
        assert not dk[b, sl, g].any() and not dv[b, sl, g].any(), f"dK/dV of unselected chunk {c}"


# ---------------------------------------------------------------------------
# fuzz: random shapes, layouts, selections and flags drawn from a seeded generator
# ---------------------------------------------------------------------------
def _fuzz_case(seed, base):
    rng = np.random.default_rng(base + seed)
    Hkv = int(rng.choice([1, 2]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    causal = bool(rng.random() < 0.4)
    kw = dict(B=int(rng.integers(1, 3)), Hq=Hq, Hkv=Hkv, Nq=int(rng.integers(1, 520)),
              Nk=int(rng.integers(1, 520)), d=int(rng.choice([64, 128])), max_qblock=int(rng.integers(1, 260)),
              max_kblock=int(rng.integers(1, 140)), density=float(rng.uniform(0.05, 0.9)),
              sel_mode=str(rng.choice(["shared", "kv", "head", "batch-kv"])), allow_empty=bool(rng.random() < 0.4),
              use_perm=bool(rng.random() < 0.4), causal=causal, unsorted=bool(rng.random() < 0.3),
              dup=bool(rng.random() < 0.3))
    if causal:
        kw["q_pos0"] = int(rng.integers(-100, 200))
    return make_random(base + 1000 + seed, **kw)


@pytest.mark.parametrize("seed", range(8))
def test_bwd_fuzz_full(seed):
    check_full(_fuzz_case(seed, 5000), f"bwd-fuzz-{seed}")
