"""Page lists rebuilt on the GPU (bsattn_plan_update_selection) against the host planner and
the float64 oracle.

A plan created with one selection and updated on the device with another must run exactly
like a plan built on the host for the second selection: the forward outputs and the
backward's gradients are compared bit for bit (same lists, same work order), and the
forward against the oracle at the forward's bar.
Error bits: capacity exceeded, block id out of range, row not ascending.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_fwd_amd as bs
from oracle.attention import masked_attention_w
from workloads.configs import make_random, make_chunk_gqa
from tests.oracle_select import oracle_chunk_select

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _canonical(w):
    """Rows sorted ascending and deduplicated (what the device update requires)."""
    rp, cols = [0], []
    for r in range(len(w.sel_row_ptr) - 1):
        row = sorted(set(int(x) for x in w.sel_kblk[w.sel_row_ptr[r]:w.sel_row_ptr[r + 1]]))
        cols.extend(row)
        rp.append(len(cols))
    return np.asarray(rp, np.int32), np.asarray(cols, np.int32)


@pytest.mark.parametrize("seed,perm,causal,decode,many_rows", [(401, False, False, False, False),
                                                               (402, True, False, False, False),
                                                               (403, False, True, False, False),
                                                               (404, False, True, True, False),
                                                               (405, False, False, False, True),
                                                               (406, False, True, True, True)])
def test_device_update_equals_host_plan(seed, perm, causal, decode, many_rows):
    # The update builds few rows with a workgroup per row and many rows (>= 256: ~1,300 rows
    # of small Q blocks) with a wave per row.  Count arrays longer than 16,384 (the decode case
    # with 5,000 chunks per sequence: 20,000 transposed lists) are scanned over the whole chip.
    if decode:
        nch = 5000 if many_rows else 120
        w1 = make_chunk_gqa("u1", seed, B=2, Hq=16, Hkv=2, d=128, Nk=64 * nch, Nq=1, chunk=64, topk=30,
                            chunk_select=oracle_chunk_select)
        w2 = make_chunk_gqa("u2", seed + 50, B=2, Hq=16, Hkv=2, d=128, Nk=64 * nch, Nq=1, chunk=64, topk=30,
                            chunk_select=oracle_chunk_select)
        w2.q, w2.k, w2.v = w1.q, w1.k, w1.v  # same tensors, the second seed's selection
    else:
        nq, mq = (3000, 8) if many_rows else (400, 130)
        w1 = make_random(seed, B=1, Hq=4, Hkv=2, Nq=nq, Nk=600, d=128, max_qblock=mq, max_kblock=50, density=0.5,
                         sel_mode="kv", use_perm=perm, causal=causal)
        w2 = make_random(seed, B=1, Hq=4, Hkv=2, Nq=nq, Nk=600, d=128, max_qblock=mq, max_kblock=50, density=0.3,
                         sel_mode="kv", use_perm=perm, causal=causal)
        rows = len(w2.sel_row_ptr) - 1
        assert (rows >= 256) == many_rows, rows
    rp2, kb2 = _canonical(w2)
    a = bs.Plan.from_workload(w1).upload()
    cap = a.stats["page_list_len"]
    b = bs.Plan.from_workload(w2).upload()
    assert b.stats["page_list_len"] <= cap, "the second selection must fit the first's capacity"
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    a.update_selection(w2.sel_nb, w2.sel_nh, _i32(rp2), _i32(kb2), status)
    q, k, v = _dev(w2.q), _dev(w2.k), _dev(w2.v)
    run = (lambda p: p.fwd_decode(q, k, v, scale=w2.scale)) if decode else (lambda p: p.fwd(q, k, v, scale=w2.scale))
    oa, la = run(a)
    ob, lb = run(b)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(oa, ob) and torch.equal(la, lb), "device-built lists differ from the host plan's"
    O = np.transpose(oa.float().cpu().numpy().astype(np.float64), (0, 2, 1, 3))
    L = la.cpu().numpy().astype(np.float64)
    Or, Lr = masked_attention_w(w2)
    Or = np.transpose(Or, (0, 2, 1, 3))
    live = np.isfinite(Lr)
    assert np.array_equal(np.isfinite(L), live)
    err = np.abs(O[live] - Or[live])
    _say(f"update seed {seed}: O max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 1e-3 and np.abs(L[live] - Lr[live]).max() <= 1e-3
    # the backward walks the device-built transposed lists: bitwise the host plan's gradients
    # (dO: any bf16 tensor in O's layout)
    ga = a.bwd(q, k, v, oa, la, q, scale=w2.scale)
    gb = b.bwd(q, k, v, ob, lb, q, scale=w2.scale)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for name, x, y in zip(("dQ", "dK", "dV"), ga, gb):
        assert torch.equal(x, y), f"{name} from the device-built lists differs from the host plan's"
    a.upload(a.device_buffer)
    oc, lc = run(a)
    o1, l1 = run(bs.Plan.from_workload(w1).upload())
    torch.cuda.synchronize()
    assert torch.equal(oc, o1) and torch.equal(lc, l1)


def test_device_update_status_bits():
    w = make_random(410, B=1, Hq=2, Hkv=2, Nq=200, Nk=300, d=64, max_qblock=64, max_kblock=40, density=0.2,
                    sel_mode="kv")
    a = bs.Plan.from_workload(w).upload()
    rows = len(w.sel_row_ptr) - 1
    nkb = w.n_kblocks
    q, k, v = _dev(w.q), _dev(w.k), _dev(w.v)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    # every block in every row: more pages than the capacity -> lists cut, bit 1
    rp = np.arange(rows + 1, dtype=np.int32) * nkb
    kb = np.tile(np.arange(nkb, dtype=np.int32), rows)
    a.update_selection(1, w.sel_nh, _i32(rp), _i32(kb), status)
    o, l = a.fwd(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    assert int(status.item()) & 1
    assert torch.isfinite(o.float()).all()
    # an id out of range and a descending row
    status.zero_()
    rp = np.array([0, 2] + [2] * (rows - 1), dtype=np.int32)
    a.update_selection(1, w.sel_nh, _i32(rp), _i32([3, nkb + 5]), status)
    torch.cuda.synchronize()
    assert int(status.item()) & 2
    status.zero_()
    a.update_selection(1, w.sel_nh, _i32(rp), _i32([3, 1]), status)
    torch.cuda.synchronize()
    assert int(status.item()) & 4


def test_chunk_select_to_decode_on_device():
    # the whole step on the device: chunk selection -> page lists -> head-stacked decode, equal
    # to the host plan built from the same chunks
    w = make_chunk_gqa("pipe", 420, B=2, Hq=16, Hkv=2, d=128, Nk=64 * 200, Nq=1, chunk=64, topk=50,
                       chunk_select=oracle_chunk_select)
    q, k, v = _dev(w.q), _dev(w.k), _dev(w.v)
    plan = bs.Plan.from_workload(w).upload()
    _, chunks = bs.chunk_select(q, k, w.Hkv, 64, 50)
    rp = torch.arange(0, w.B * w.Hkv * 50 + 1, 50, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan.update_selection(w.B, w.Hkv, rp, chunks.reshape(-1).contiguous(), status)
    o1, l1 = plan.fwd_decode(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    w.sel_kblk = chunks.cpu().numpy().reshape(-1).astype(np.int32)
    o2, l2 = bs.Plan.from_workload(w).upload().fwd_decode(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
