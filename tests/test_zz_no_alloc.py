"""GPU: the allocation-free decode (bsattn_fwd_decode_noalloc, partial states in the
library's own device buffer) against the workspace decode (bsattn_fwd_decode) on the same
plan, through the C ABI: bitwise the same outputs, and within the forward's bar of the
float64 oracle.  Two calls in a row, the second on a smaller problem, so the second reads
only what it wrote over the first call's states."""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_fwd_amd as bs
from oracle.attention import masked_attention_w
from workloads.configs import make_chunk_gqa
from tests.oracle_select import oracle_chunk_select

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def _decode_both(w):
    plan = bs.Plan.from_workload(w).upload()
    q, k, v = _dev(w.q), _dev(w.k), _dev(w.v)
    outs = []
    for noalloc in (True, False):
        o = torch.full((w.B, w.Nq, w.Hq, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((w.B, w.Hq, w.Nq), float("nan"), dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        if noalloc:
            bs.bsattn_fwd_decode_noalloc(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                         lse.data_ptr(), float(w.scale), stream)
        else:
            nws = bs.bsattn_decode_workspace_bytes(plan.handle)
            ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
            bs.bsattn_fwd_decode(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 float(w.scale), ws.data_ptr(), nws, stream)
        torch.cuda.synchronize()
        outs.append((o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)))
    return outs


def test_noalloc_decode_two_calls():
    cases = [
        make_chunk_gqa("decode-a", 401, B=2, Hq=16, Hkv=2, d=128, Nk=64 * 300, Nq=2, chunk=64, topk=120,
                       chunk_select=oracle_chunk_select),
        make_chunk_gqa("decode-b", 402, B=1, Hq=8, Hkv=1, d=128, Nk=64 * 90, Nq=1, chunk=64, topk=30,
                       chunk_select=oracle_chunk_select),
    ]
    for w in cases:
        print(f"[noalloc] {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk}", flush=True)
        (o1, l1), (o2, l2) = _decode_both(w)
        assert np.all(np.isfinite(o1))
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        Or, Lr = masked_attention_w(w)
        O = np.transpose(o1, (0, 2, 1, 3))
        Or = np.transpose(Or, (0, 2, 1, 3))
        live = np.isfinite(Lr)
        assert np.array_equal(np.isfinite(l1), live)
        err = np.abs(O[live] - Or[live])
        lerr = np.abs(l1[live] - Lr[live])
        print(f"[noalloc] {w.name}: O max {err.max():.3e} mean {err.mean():.3e}; LSE max {lerr.max():.3e}", flush=True)
        assert err.max() <= 2e-2 and err.mean() <= 1e-3 and lerr.max() <= 1e-3
