"""GPU parity of the head-stacked decode path (bsattn_fwd_decode) against the float64 oracle.

Same bar as the forward: O max-abs <= 2e-2, mean-abs <= 1e-3, LSE max-abs <= 1e-3 on rows
with keys; rows without keys exactly O = 0 and LSE = -inf.  Every output is compared.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_fwd_amd as bs
from oracle.attention import masked_attention_w
from workloads.configs import make_chunk_gqa, make_random
from tests.oracle_select import oracle_chunk_select

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def check_decode(w, label):
    _say(f"[gpu-decode] {label}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d} causal={w.causal}")
    plan = bs.Plan.from_workload(w).upload()
    q, k, v = _dev(w.q), _dev(w.k), _dev(w.v)
    o = torch.full((w.B, w.Nq, w.Hq, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.B, w.Hq, w.Nq), float("nan"), dtype=torch.float32, device="cuda")
    plan.fwd_decode(q, k, v, o, lse, scale=w.scale)
    torch.cuda.synchronize()
    O = np.transpose(o.float().cpu().numpy().astype(np.float64), (0, 2, 1, 3))
    L = lse.cpu().numpy().astype(np.float64)
    Or, Lr = masked_attention_w(w)
    Or = np.transpose(Or, (0, 2, 1, 3))
    assert np.all(np.isfinite(O)), f"{label}: unwritten or non-finite O"
    live = np.isfinite(Lr)
    assert np.array_equal(np.isfinite(L), live), f"{label}: LSE finiteness differs"
    assert np.all(O[~live] == 0.0) and np.all(L[~live] == -np.inf)
    if live.any():
        err = np.abs(O[live] - Or[live])
        lerr = np.abs(L[live] - Lr[live])
        _say(f"{label}: O max {err.max():.3e} mean {err.mean():.3e}; LSE max {lerr.max():.3e}")
        assert err.max() <= 2e-2 and err.mean() <= 1e-3 and lerr.max() <= 1e-3


@pytest.mark.parametrize("Nq,Hq,Hkv,d", [(1, 16, 2, 128), (4, 16, 2, 128), (2, 8, 8, 128), (1, 8, 1, 64)])
def test_decode_chunk_gqa(Nq, Hq, Hkv, d):
    w = make_chunk_gqa("decode", 300 + Nq + d, B=2, Hq=Hq, Hkv=Hkv, d=d, Nk=64 * 150 + 64, Nq=Nq, chunk=64, topk=40,
                       chunk_select=oracle_chunk_select)
    check_decode(w, f"chunk-gqa Nq={Nq} Hq={Hq} Hkv={Hkv} d={d}")


@pytest.mark.parametrize("seed,perm,causal", [(311, False, False), (312, True, False), (313, True, True),
                                              (314, False, True)])
def test_decode_random_small_blocks(seed, perm, causal):
    # many Q blocks of 1-4 rows, grouped heads sharing a selection per KV group, empty blocks
    w = make_random(seed, B=2, Hq=8, Hkv=2, Nq=90, Nk=700, d=128, max_qblock=4, max_kblock=60, density=0.4,
                    sel_mode="kv", use_perm=perm, causal=causal, allow_empty=True)
    check_decode(w, f"random-{seed}")


def test_decode_matches_forward_path():
    w = make_chunk_gqa("decode", 320, B=1, Hq=16, Hkv=2, d=128, Nk=64 * 300, Nq=2, chunk=64, topk=100,
                       chunk_select=oracle_chunk_select)
    plan = bs.Plan.from_workload(w).upload()
    q, k, v = _dev(w.q), _dev(w.k), _dev(w.v)
    o1, l1 = plan.fwd(q, k, v, scale=w.scale)
    o2, l2 = plan.fwd_decode(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
    assert (l1 - l2).abs().max().item() <= 1e-4
