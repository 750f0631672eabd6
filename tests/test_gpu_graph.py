"""HIP-graph capture of the C-ABI calls: the forward, the backward and the head-stacked decode
allocate nothing and clear nothing with memsets, so a caller can record them into a graph
and replay it.  Every replay is compared bitwise with the eager result of the same call on
the same inputs, with eager work and synchronisations between the replays; the eager
results themselves are checked against the float64 oracle."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import block_sparse_attention_fwd_amd as bs  # noqa: E402
from oracle.attention import masked_attention_w  # noqa: E402
from workloads.configs import draw_dout, make_chunk_gqa, make_random  # noqa: E402
from tests.oracle_select import oracle_chunk_select  # noqa: E402

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def _replays_match(g, outs, eager, label, n=3):
    for r in range(n):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outs, eager)):
            assert torch.equal(t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32),
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e.view(torch.int32)), \
                f"{label}: replay {r}, output {i} differs from the eager call"
        # eager work between replays
        torch.ones(1 << 20, device="cuda").sum().item()
    _say(f"[gpu-graph] {label}: {n} replays bitwise equal to the eager call")


def test_graph_forward_backward():
    w = make_random(501, B=1, Hq=4, Hkv=2, Nq=600, Nk=700, d=128, max_qblock=200, max_kblock=60, sel_mode="kv",
                    causal=True, q_pos0=100, density=0.4)
    _say(f"[gpu-graph] forward + backward: Nq={w.Nq} Nk={w.Nk} d={w.d}")
    plan = bs.Plan.from_workload(w).upload()
    q, k, v, do = _dev(w.q), _dev(w.k), _dev(w.v), _dev(draw_dout(w))
    o = torch.empty((w.B, w.Nq, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nws = bs.bsattn_bwd_workspace_bytes(plan.handle)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def step(stream):
        bs.bsattn_fwd(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      float(w.scale), stream)
        bs.bsattn_bwd(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), float(w.scale), ws.data_ptr(), nws,
                      stream)

    step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o, lse, dq, dk, dv)]
    # the eager forward against the oracle
    Or, Lr = masked_attention_w(w)
    O = eager[0].float().cpu().numpy().astype(np.float64)
    live = np.isfinite(Lr)
    err = np.abs(np.transpose(O, (0, 2, 1, 3))[live] - np.transpose(Or, (0, 2, 1, 3))[live])
    assert err.max() <= 2e-2 and err.mean() <= 1e-3

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    _replays_match(g, [o, lse, dq, dk, dv], eager, "forward + backward")


def test_graph_decode():
    w = make_chunk_gqa("graph-decode", 502, B=2, Hq=16, Hkv=2, d=128, Nk=64 * 120, Nq=1, chunk=64, topk=40,
                       chunk_select=oracle_chunk_select)
    _say(f"[gpu-graph] decode: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nk={w.Nk}")
    plan = bs.Plan.from_workload(w).upload()
    q, k, v = _dev(w.q), _dev(w.k), _dev(w.v)
    o = torch.empty((w.B, w.Nq, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
    nws = bs.bsattn_decode_workspace_bytes(plan.handle)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def step(stream):
        bs.bsattn_fwd_decode(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             float(w.scale), ws.data_ptr(), nws, stream)

    step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    eager = [o.clone(), lse.clone()]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    _replays_match(g, [o, lse], eager, "decode")
