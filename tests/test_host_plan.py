"""Host planner of libbsattn against the oracle's plan, bit for bit (CPU only; no GPU call).

The planner is host C++ inside libbsattn.so; these tests create plans and read them
back through the C ABI (bsattn_plan_create / _stats / _export) and compare every array
and count with oracle.planner.  Nothing here launches a kernel.
"""
import ctypes
import subprocess

import numpy as np
import pytest

import block_sparse_attention_fwd_amd as bs
from oracle.planner import build_plan_w, build_bwd_plan_w
from workloads.configs import make, make_random, make_chunk_gqa
from tests.oracle_select import oracle_chunk_select


def _compare(w, flags=0):
    p = bs.Plan.from_workload(w, flags=flags)
    ex = p.export()
    st = p.stats
    o = build_plan_w(w, fixed_tiles=bool(flags & bs.PLAN_FIXED_TILES))
    for name in ("page_kblock", "page_slot0", "page_nvalid", "qt_qblock", "qt_row0", "qt_rows", "qt_shape",
                 "pl_ptr", "pl_pages"):
        assert np.array_equal(ex[name], getattr(o, name)), name
    assert st["useful"] == o.useful
    assert st["physical"] == o.physical
    assert st["n_ktiles"] == o.n_ktiles
    assert st["n_pages"] == o.n_pages
    assert (st["n_qtiles128"], st["n_qtiles64"]) == (o.n_qtiles128, o.n_qtiles64)
    assert st["page_list_len"] == len(o.pl_pages)
    assert tuple(st["physical_by_shape"]) == o.physical_by_shape
    assert tuple(st["useful_by_shape"]) == o.useful_by_shape
    assert sum(o.useful_by_shape) == o.useful
    eb = p.export_bwd()
    ob = build_bwd_plan_w(w)
    for name in ("qpage_qblock", "qpage_slot0", "qpage_nvalid", "dqt_qblock", "dqt_row0", "dqt_rows", "kvt_kblock",
                 "kvt_row0", "kvt_rows", "tpl_ptr", "tpl_pages"):
        assert np.array_equal(eb[name], getattr(ob, name)), name
    return st


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_configs_bit_exact(cfg):
    _compare(make(cfg, with_tensors=False))


def test_chunk_gqa_scaled_bit_exact():
    w = make_chunk_gqa("small", 5, B=2, Hq=8, Hkv=2, d=64, Nk=64 * 300, Nq=512, chunk=64, topk=120,
                       chunk_select=oracle_chunk_select)
    st = _compare(w)
    assert st["useful"] < 2 * 8 * 512 * 120 * 64  # causal exclusions removed


@pytest.mark.parametrize("cfg", [1, 3, 4])
def test_fixed_tiles_bit_exact(cfg):
    _compare(make(cfg, with_tensors=False), flags=bs.PLAN_FIXED_TILES)


def test_unknown_plan_flag_is_arg_error():
    w = make_random(5, Nq=40, Nk=40, d=64, with_tensors=False)
    with pytest.raises(bs.BsattnError) as e:
        bs.Plan.from_workload(w, flags=2)
    assert e.value.status == 1


@pytest.mark.parametrize("seed", range(12))
def test_random_bit_exact(seed):
    rng = np.random.default_rng(1000 + seed)
    Hkv = int(rng.choice([1, 2]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    kw = dict(B=int(rng.integers(1, 3)), Hq=Hq, Hkv=Hkv, Nq=int(rng.integers(1, 700)),
              Nk=int(rng.integers(1, 700)), d=64, max_qblock=int(rng.integers(1, 300)),
              max_kblock=int(rng.integers(1, 90)), density=float(rng.uniform(0.05, 0.9)),
              sel_mode=str(rng.choice(["shared", "kv", "head", "batch-kv"])), allow_empty=bool(rng.random() < 0.4),
              use_perm=bool(rng.random() < 0.4), causal=bool(rng.random() < 0.4), unsorted=bool(rng.random() < 0.3),
              dup=bool(rng.random() < 0.3), with_tensors=False)
    _compare(make_random(2000 + seed, **kw), flags=int(rng.random() < 0.3))


def _problem(B=1, Hq=1, Hkv=1, Nq=4, Nk=4, d=64):
    pr = bs.Problem()
    pr.B, pr.Hq, pr.Hkv, pr.Nq, pr.Nk, pr.d = B, Hq, Hkv, Nq, Nk, d
    pr.dtype = 1
    return pr


def _arr(x):
    a = np.ascontiguousarray(x, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _status(pr, qo, ko, rp, kb, qperm=None, nb=1, nh=1, page=16):
    keep = []

    def p(x):
        if x is None:
            return None
        a, ptr = _arr(x)
        keep.append(a)
        return ptr

    ql = bs.Layout(len(qo) - 1, p(qo), p(qperm))
    kl = bs.Layout(len(ko) - 1, p(ko), None)
    sel = bs.Selection(nb, nh, p(rp), p(kb))
    h = ctypes.c_void_p()
    st = bs.library().bsattn_plan_create(ctypes.byref(pr), ctypes.byref(ql), ctypes.byref(kl), ctypes.byref(sel),
                                         page, ctypes.byref(h))
    if st == 0:
        bs.library().bsattn_plan_destroy(h)
    else:
        assert not h.value
    return st


def test_error_statuses():
    ok = dict(qo=[0, 4], ko=[0, 4], rp=[0, 1], kb=[0])
    assert _status(_problem(), **ok) == 0
    assert _status(_problem(d=96), **ok) == 4                    # head_dim
    assert _status(_problem(), page=8, **ok) == 4                # page size
    assert _status(_problem(Hq=3, Hkv=2), **ok) == 1             # Hq not a multiple of Hkv
    assert _status(_problem(), qo=[0, 3], ko=[0, 4], rp=[0, 1], kb=[0]) == 2        # offsets end != Nq
    assert _status(_problem(), qo=[0, 3, 2, 4], ko=[0, 4], rp=[0, 1, 1, 1], kb=[0]) == 2  # falling offsets
    assert _status(_problem(), qperm=[0, 1, 1, 2], **ok) == 2    # not a permutation
    assert _status(_problem(), qo=[0, 4], ko=[0, 4], rp=[0, 1], kb=[1]) == 3        # block id out of range
    assert _status(_problem(), qo=[0, 4], ko=[0, 4], rp=[1, 1], kb=[0]) == 3        # row_ptr[0] != 0
    assert _status(_problem(), qo=[0, 4], ko=[0, 4], rp=[0, 1], kb=[0], nh=3) == 3  # n_h not 1/Hkv/Hq
    pr = _problem()
    pr.dtype = 2
    assert _status(pr, **ok) == 4
    h = ctypes.c_void_p()
    assert bs.library().bsattn_plan_create(None, None, None, None, 16, ctypes.byref(h)) == 1
    assert bs.bsattn_status_string(3) == "invalid block selection"


def test_fwd_before_upload_is_state_error():
    w = make_random(3, Nq=40, Nk=40, d=64, with_tensors=False)
    p = bs.Plan.from_workload(w)
    with pytest.raises(bs.BsattnError) as e:
        bs.bsattn_fwd(p.handle, 16, 16, 16, 16, 16, 0.125, 0)
    assert e.value.status == 7
    with pytest.raises(bs.BsattnError) as e:
        bs.bsattn_plan_upload(p.handle, 0, 1 << 20, 0)
    assert e.value.status == 1
    with pytest.raises(bs.BsattnError) as e:
        bs.bsattn_plan_upload(p.handle, 256, 1, 0)  # too small: rejected before any HIP call
    assert e.value.status == 1


def test_bwd_before_upload_is_state_error_and_workspace_size():
    w = make_random(4, B=2, Hq=4, Hkv=2, Nq=40, Nk=50, d=64, with_tensors=False)
    p = bs.Plan.from_workload(w)
    # D = rowsum(dO * O): float32 [B, Hq, Nq], rounded up to 256 bytes
    assert bs.bsattn_bwd_workspace_bytes(p.handle) == 1280
    with pytest.raises(bs.BsattnError) as e:
        bs.bsattn_bwd(p.handle, 16, 16, 16, 16, 16, 16, 16, 16, 16, 0.125, 256, 1 << 20, 0)
    assert e.value.status == 7


def test_library_exports_every_declared_symbol():
    import re
    import os
    hdr = open(os.path.join(os.path.dirname(bs.__file__), "..", "include", "bsattn.h")).read()
    declared = sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(bsattn_\w+)\(", hdr, re.M)))
    assert declared == sorted(bs.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", bs.LIB_PATH], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared:
        assert name in syms, name
        assert hasattr(bs.library(), name)


def test_mfma_probe_argument_errors():
    # rejected before anything touches the GPU: null or misaligned clock buffer, no
    # iterations, a grid outside 1..65535 workgroups
    lib = bs.library()
    assert lib.bsattn_mfma_probe(512, 10, 1, None, None) == 1
    assert lib.bsattn_mfma_probe(512, 10, 1, ctypes.c_void_p(12), None) == 1
    assert lib.bsattn_mfma_probe(512, 0, 1, ctypes.c_void_p(256), None) == 1
    assert lib.bsattn_mfma_probe(0, 10, 1, ctypes.c_void_p(256), None) == 1
    assert lib.bsattn_mfma_probe(65536, 10, 1, ctypes.c_void_p(256), None) == 1


def test_chunk_select_argument_errors():
    def st(**kw):
        pr = bs.ChunkProblem()
        base = dict(B=1, Hq=4, Hkv=2, Nq=8, Nk=640, d=128, chunk=64, topk=4, query_index=7, reserved=0)
        base.update(kw)
        for k, v in base.items():
            setattr(pr, k, v)
        pr.q_stride[:] = (8 * 4 * 128, 4 * 128, 128)
        pr.k_stride[:] = (640 * 2 * 128, 2 * 128, 128)
        return bs.library().bsattn_chunk_select(ctypes.byref(pr), ctypes.c_void_p(256), ctypes.c_void_p(256),
                                                ctypes.c_void_p(256), ctypes.c_void_p(256), None)
    assert st(topk=11) == 1               # more than ceil(640 / 64) = 10 chunks
    assert st(topk=0) == 1
    assert st(query_index=8) == 1
    assert st(Hq=3) == 1
    assert st(d=96) == 4
    assert st(Nk=64 * 8193, topk=4) == 4  # more than 8192 chunks
    assert bs.library().bsattn_chunk_select(None, None, None, None, None, None) == 1


def test_block_order_hint_validates_and_keeps_canonical_arrays():
    w = make(3, with_tensors=False)
    a = bs.Plan.from_workload(w, block_order=False)
    b = bs.Plan.from_workload(w)  # the cube workload's (h, t, w) hint
    for k, v in a.export().items():
        assert np.array_equal(v, b.export()[k]), k
    assert a.stats["physical"] == b.stats["physical"]
    assert sorted(w.q_block_order.tolist()) == list(range(w.n_qblocks))
    with pytest.raises(bs.BsattnError):
        a.set_block_order(np.zeros(w.n_qblocks, np.int32))        # not a permutation
    with pytest.raises(bs.BsattnError):
        a.set_block_order(np.arange(w.n_qblocks - 1, dtype=np.int32))  # wrong length


def test_decode_geometry_and_unsupported_plans():
    w = make_chunk_gqa("decode", 7, B=2, Hq=16, Hkv=2, d=128, Nk=64 * 150, Nq=1, chunk=64, topk=40,
                       chunk_select=oracle_chunk_select)
    p = bs.Plan.from_workload(w)
    assert bs.bsattn_decode_workspace_bytes(p.handle) > 0
    big = make_random(8, B=1, Hq=8, Hkv=1, Nq=100, Nk=100, d=64, max_qblock=20, sel_mode="kv", with_tensors=False)
    pb = bs.Plan.from_workload(big)  # Q blocks of up to 20 rows x 8 heads > 32 columns
    with pytest.raises(bs.BsattnError) as e:
        bs.bsattn_decode_workspace_bytes(pb.handle)
    assert e.value.status == 4
    per_head = make_random(9, B=1, Hq=4, Hkv=2, Nq=20, Nk=100, d=64, max_qblock=4, sel_mode="head",
                           with_tensors=False)
    ph = bs.Plan.from_workload(per_head)  # held: a temporary Plan is destroyed before the call
    with pytest.raises(bs.BsattnError) as e:
        bs.bsattn_decode_workspace_bytes(ph.handle)
    assert e.value.status == 4


def test_decode_noalloc_limits():
    # the allocation-free decode holds its partial states in a 16 MiB library buffer: plans
    # needing more are rejected before anything touches a GPU, and so are plans the decode
    # path does not take; a fitting plan that was never uploaded is a state error
    many = make_random(21, B=1, Hq=8, Hkv=8, Nq=420, Nk=64, d=128, max_qblock=4, max_kblock=16, sel_mode="kv",
                       density=0.5, with_tensors=False)
    pm = bs.Plan.from_workload(many)
    assert bs.bsattn_decode_workspace_bytes(pm.handle) > 16 << 20
    with pytest.raises(bs.BsattnError) as e:
        bs.bsattn_fwd_decode_noalloc(pm.handle, 16, 16, 16, 16, 16, 0.125, 0)
    assert e.value.status == 4
    big = make_random(8, B=1, Hq=8, Hkv=1, Nq=100, Nk=100, d=64, max_qblock=20, sel_mode="kv", with_tensors=False)
    pb = bs.Plan.from_workload(big)
    with pytest.raises(bs.BsattnError) as e:
        bs.bsattn_fwd_decode_noalloc(pb.handle, 16, 16, 16, 16, 16, 0.125, 0)
    assert e.value.status == 4
    w = make_chunk_gqa("decode", 7, B=2, Hq=16, Hkv=2, d=128, Nk=64 * 150, Nq=1, chunk=64, topk=40,
                       chunk_select=oracle_chunk_select)
    p = bs.Plan.from_workload(w)
    assert bs.bsattn_decode_workspace_bytes(p.handle) <= 16 << 20
    with pytest.raises(bs.BsattnError) as e:
        bs.bsattn_fwd_decode_noalloc(p.handle, 16, 16, 16, 16, 16, 0.125, 0)
    assert e.value.status == 7


def test_update_selection_needs_upload():
    w = make_random(12, B=1, Hq=2, Hkv=2, Nq=40, Nk=40, d=64, sel_mode="kv", with_tensors=False)
    p = bs.Plan.from_workload(w)
    with pytest.raises(bs.BsattnError) as e:
        bs.bsattn_plan_update_selection(p.handle, w.sel_nb, w.sel_nh, 256, 256)
    assert e.value.status == 7


# Property-based sweep of the same bit-exact comparison: hypothesis draws the problem shape,
# the layouts (block sizes, empty blocks, permutations), the selection (density, sharing
# mode, unsorted rows with duplicates), causality and the plan flags.
from hypothesis import given, settings, HealthCheck, strategies as hst  # noqa: E402


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow], derandomize=True)
@given(seed=hst.integers(0, 1 << 20), B=hst.integers(1, 2), Hkv=hst.sampled_from([1, 2]),
       grp=hst.sampled_from([1, 2, 4]), Nq=hst.integers(1, 500), Nk=hst.integers(1, 500),
       d=hst.sampled_from([64, 128]), max_qblock=hst.integers(1, 300), max_kblock=hst.integers(1, 140),
       density=hst.floats(0.02, 1.0), sel_mode=hst.sampled_from(["shared", "kv", "head", "batch-kv"]),
       allow_empty=hst.booleans(), use_perm=hst.booleans(), causal=hst.booleans(), unsorted=hst.booleans(),
       dup=hst.booleans(), fixed=hst.booleans())
def test_property_bit_exact(seed, B, Hkv, grp, Nq, Nk, d, max_qblock, max_kblock, density, sel_mode, allow_empty,
                            use_perm, causal, unsorted, dup, fixed):
    w = make_random(seed, B=B, Hq=Hkv * grp, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, max_qblock=max_qblock,
                    max_kblock=max_kblock, density=density, sel_mode=sel_mode, allow_empty=allow_empty,
                    use_perm=use_perm, causal=causal, unsorted=unsorted, dup=dup, with_tensors=False)
    st = _compare(w, flags=bs.PLAN_FIXED_TILES if fixed else 0)
    assert st["physical"] >= st["useful"] >= 0
