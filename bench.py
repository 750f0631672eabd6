#!/usr/bin/env python3
"""Benchmark: exact block-sparse attention forward on one MI355X.

A step is one forward pass over the whole workload: one ``bsattn_fwd`` call, which runs
the 128x128 and 64x256 tiles in one kernel launch.  With ``--split-shapes`` the two shapes
are launched one after the other instead (``bsattn_fwd_shape``, HIP events between them),
to time each shape's tiles.  Inputs are seeded synthetic bf16 tensors already resident in
HBM; the plan is built and uploaded before timing.

Metric: useful-pair TFLOP/s = 4 * d * (query-key pairs of the sparse graph) / step time.
The default workload is the video-DiT 3D partial-block case (latent grid 21x45x80,
cubes 2x8x8, 40 heads, d = 128, sliding-tile window +-1 t, +-2 h, +-2 w in cube units).

With ``--fixed-tiles`` the plan is the fixed-tile baseline (one 128x128 tile per selected
block pair, no page packing, no 64x256 routing) -- the ablation of packing on the same
kernels.  With ``--decode`` a step is one ``bsattn_fwd_decode`` call (one query per
sequence, the query heads of a KV group stacked; HBM-bound, GB/s), with the plain forward
over the same plan timed beside it.  With ``--chunk-select`` a step is one ``bsattn_chunk_select`` call (chunk
summaries and top-k chunks of the chunk-indexed prefill workload; HBM-bound, reported in
GB/s).  With ``--bwd`` a step is one ``bsattn_bwd`` call (D = rowsum(dO * O), then the dK/dV and dQ
kernels) on the independent Q/K partition workload, counted as 10 * d per useful pair.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
SHORT_NAMES = {1: "tiny3d", 2: "onedim", 3: "videodit3d", 4: "partitions", 5: "chunkgqa"}
KERNEL_SRC = os.path.join(ROOT, "block_sparse_attention_fwd_amd", "csrc", "fwd_kernel.hip")
DECODE_SRC = os.path.join(ROOT, "block_sparse_attention_fwd_amd", "csrc", "decode_kernel.hip")
CHUNK_SRC = os.path.join(ROOT, "block_sparse_attention_fwd_amd", "csrc", "chunk_select.hip")
BWD_SRC = os.path.join(ROOT, "block_sparse_attention_fwd_amd", "csrc", "bwd_kernel.hip")


def measured_counters(workload, name=None, src=KERNEL_SRC):
    """Per-launch figures recorded by rocprofv3 counter runs in profiles/traffic_<name>.txt
    (key = value lines; name defaults to the workload's short name), or {} unless the kernel
    source src is the one measured."""
    import hashlib
    name = name or SHORT_NAMES.get(workload, "")
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
    if not os.path.exists(path):
        return {}
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    return kv if kv.get("source_sha256") == sha else {}


def measured_bytes(name, src, tags):
    """HBM bytes per call (read + write, summed over the kernels tagged) from the counter runs
    in profiles/traffic_<name>.txt, or None unless src is the source measured."""
    kv = measured_counters(None, name, src)
    try:
        return sum(int(kv[f"{t}.read_bytes"]) + int(kv[f"{t}.write_bytes"]) for t in tags)
    except KeyError:
        return None


def measured_traffic(workload, shape_tag):
    """HBM bytes per launch (read + write) from the counter runs, or None."""
    kv = measured_counters(workload)
    try:
        return int(kv[f"{shape_tag}.read_bytes"]) + int(kv[f"{shape_tag}.write_bytes"])
    except KeyError:
        return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(w, seconds):
    """The float64 oracle, as it stands, on a bounded sample of the same workload: the
    first query rows of (batch 0, head 0), 256 at a time, until ``seconds`` have passed."""
    from oracle.attention import masked_attention_w, token_block_map, token_mask
    cores = len(os.sched_getaffinity(0))
    bq = token_block_map(w.q_offsets, w.q_perm, w.Nq)
    bk = token_block_map(w.k_offsets, w.k_perm, w.Nk)
    useful = 0
    rows = 0
    t_total = 0.0
    while t_total < seconds and rows < w.Nq:
        toks = np.arange(rows, min(rows + 256, w.Nq))
        t0 = time.perf_counter()
        masked_attention_w(w, rows=[(0, 0, toks)])
        t_total += time.perf_counter() - t0
        m = token_mask(bq, bk, w.sel_row_ptr, w.sel_kblk, 0, w.n_qblocks, w.n_kblocks, toks, w.causal, w.q_pos0)
        useful += int(m.sum())
        rows += len(toks)
    tflops = 4.0 * w.d * useful / t_total / 1e12
    return {"value": tflops, "unit": "useful-pair TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 masked dense oracle on query tokens 0..{rows - 1} of batch 0, head 0 "
                      f"({useful} useful pairs, {t_total:.1f} s)"}


def cpu_baseline_bwd(w, do, seconds):
    """The float64 backward oracle, as it stands, on a bounded sample: dQ of the first query
    rows of (batch 0, head 0), 256 at a time, until ``seconds`` have passed.  Each such row
    costs the oracle its scores, probabilities, O, D, dP, dS and dQ over the full key width;
    the rate counts 10*d per useful pair of the sampled rows."""
    from oracle.attention import masked_attention_bwd_w, token_block_map, token_mask
    cores = len(os.sched_getaffinity(0))
    bq = token_block_map(w.q_offsets, w.q_perm, w.Nq)
    bk = token_block_map(w.k_offsets, w.k_perm, w.Nk)
    useful = rows = 0
    t_total = 0.0
    while t_total < seconds and rows < w.Nq:
        toks = np.arange(rows, min(rows + 256, w.Nq))
        t0 = time.perf_counter()
        masked_attention_bwd_w(w, do, q_rows=[(0, 0, toks)])
        t_total += time.perf_counter() - t0
        m = token_mask(bq, bk, w.sel_row_ptr, w.sel_kblk, 0, w.n_qblocks, w.n_kblocks, toks, w.causal, w.q_pos0)
        useful += int(m.sum())
        rows += len(toks)
    return {"value": 10.0 * w.d * useful / t_total / 1e12, "unit": "useful-pair TFLOP/s (10*d per pair)",
            "cores": cores, "kind": "oracle",
            "sample": f"float64 backward oracle, dQ of query tokens 0..{rows - 1} of batch 0, head 0 "
                      f"({useful} useful pairs, {t_total:.1f} s; the dK/dV products are not in the sample)"}


def cpu_baseline_chunks(w, chunk, topk, gpu_chunks):
    """The float64 oracle's chunk selection, as it stands, on batch 0 (every KV group): mean-key
    summaries, indexing queries, scores and the top-k, in GB/s of K read; also whether it picks
    the same chunks as the GPU did for that batch."""
    from oracle.chunk_index import chunk_scores, select_chunks
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    ref = select_chunks(chunk_scores(w.q[:1], w.k[:1], chunk, w.Hkv, w.Nq - 1), topk)
    t = time.perf_counter() - t0
    same = bool(np.array_equal(np.asarray(ref).reshape(w.Hkv, topk), gpu_chunks[0].reshape(w.Hkv, topk)))
    nbytes = w.Nk * w.Hkv * w.d * 2
    return {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 chunk selection oracle on batch 0 ({w.Hkv} KV groups, {w.Nk} keys, {t:.1f} s); "
                      f"same chunks as the GPU: {same}"}


def gpu_chunk_select(w, chunk, topk):
    """Selection of the chunk-indexed workloads (chunk summaries scored by one indexing query
    per KV group, top-k) computed on the GPU by bsattn_chunk_select from the drawn Q and K;
    the GPU tests check that call against the float64 oracle."""
    import torch
    import block_sparse_attention_fwd_amd as bs

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda:0")

    q, k = to_dev(w.q), to_dev(w.k)
    _, chunks = bs.chunk_select(q, k, w.Hkv, chunk, topk)
    torch.cuda.synchronize()
    sel = chunks.cpu().numpy().astype(np.int32).reshape(w.B * w.Hkv, topk)
    del q, k
    return sel


def bench_bwd(args, w, plan, st, t_plan, dev):
    """One step = one bsattn_bwd call (D, then dK/dV, then dQ) on resident inputs, with O and
    LSE from one forward call before the timed region."""
    import torch
    import block_sparse_attention_fwd_amd as bs
    from workloads.configs import draw_dout

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    do_np = draw_dout(w)
    q, k, v, do = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(do_np)
    o, lse = plan.fwd(q, k, v, scale=w.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nws = bs.bsattn_bwd_workspace_bytes(plan.handle)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), float(w.scale), ws.data_ptr(), nws, stream.cuda_stream)
    for _ in range(args.warmup):
        bs.bsattn_bwd(plan.handle, *ptrs)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        events[i][0].record(stream)
        bs.bsattn_bwd(plan.handle, *ptrs)
        events[i][1].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    log(f"[bench] backward {ms_step:.3f} ms/step (wall), {ev_ms:.3f} ms (events)")
    flop = 10.0 * w.d * st["useful"]
    value = flop / (ms_step * 1e-3) / 1e12
    achieved = flop / (ev_ms * 1e-3) / 1e12
    cpu = None
    if args.cpu_seconds > 0:
        log(f"[bench] timing the CPU backward oracle for about {args.cpu_seconds:.0f} s")
        cpu = cpu_baseline_bwd(w, do_np, args.cpu_seconds)
    out = {
        "metric": "useful-pair backward TFLOP/s (10*d*valid QK pairs/s), % bf16 MFMA peak, 1 GPU",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V/dO; block layout and selection as the workload defines)",
        "config": {"workload": w.name, "pass": "backward", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq,
                   "Nk": w.Nk, "d": w.d, "useful_pairs": st["useful"],
                   "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2), "plan_ms": round(t_plan * 1e3, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     # HBM bytes of one backward call (all its kernels) from the committed counter runs
                     "traffic": measured_bytes(f"bwd_{SHORT_NAMES.get(args.workload, '')}", BWD_SRC,
                                               ("bwd_dot_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel",
                                                "bwd_dq_kernel_split")),
                     "kernel": f"bsattn_bwd: bwd_dot + bwd_dkdv<{w.d}> + bwd_dq<{w.d}>", "kernel_ms": round(ev_ms, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_chunk_select(args, w, dev):
    """One step = one bsattn_chunk_select call (chunk summaries, then the top-k per
    (batch, KV group)) on the chunk-indexed prefill shapes; HBM-bound: K is read once."""
    import torch
    import block_sparse_attention_fwd_amd as bs

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    chunk, topk = int(w.k_offsets[1] - w.k_offsets[0]), int(w.sel_row_ptr[1] - w.sel_row_ptr[0])
    q, k = to_dev(w.q), to_dev(w.k)
    summ, chunks = bs.chunk_select(q, k, w.Hkv, chunk, topk)
    torch.cuda.synchronize()
    pr = bs.ChunkProblem()
    pr.B, pr.Hq, pr.Hkv, pr.Nq, pr.Nk, pr.d = w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d
    pr.chunk, pr.topk, pr.query_index, pr.reserved = chunk, topk, w.Nq - 1, 0
    pr.q_stride[:] = tuple(q.stride()[:3])
    pr.k_stride[:] = tuple(k.stride()[:3])
    stream = torch.cuda.current_stream()
    ptrs = (q.data_ptr(), k.data_ptr(), summ.data_ptr(), chunks.data_ptr(), stream.cuda_stream)
    for _ in range(args.warmup):
        bs.bsattn_chunk_select(pr, *ptrs)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        events[i][0].record(stream)
        bs.bsattn_chunk_select(pr, *ptrs)
        events[i][1].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    n = summ.shape[2]
    # algorithmic bytes: K once, the summaries written and read back once, the chunk ids
    nbytes = w.B * w.Nk * w.Hkv * w.d * 2 + 2 * w.B * w.Hkv * n * w.d * 4 + w.B * w.Hkv * topk * 4
    log(f"[bench] chunk selection {ms_step:.3f} ms/step (wall), {ev_ms:.3f} ms (events)")
    cpu = None
    if args.cpu_seconds > 0:
        log("[bench] timing the CPU oracle's chunk selection on batch 0")
        cpu = cpu_baseline_chunks(w, chunk, topk, chunks.cpu().numpy())
    out = {
        "metric": "chunk selection HBM GB/s (K read once + summaries), 1 GPU",
        "value": round(nbytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K)",
        "config": {"workload": w.name, "pass": "chunk selection", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq,
                   "Nk": w.Nk, "d": w.d, "chunk": chunk, "topk": topk, "n_chunks": n, "bytes": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (ev_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(nbytes / (ev_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": measured_bytes("chunkselect", CHUNK_SRC, ("chunk_summary_kernel", "chunk_topk_kernel")),
                     "kernel": f"chunk_summary_kernel<{w.d}> + chunk_topk_kernel<{w.d}>", "kernel_ms": round(ev_ms, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_decode(args, dev):
    """One step = one bsattn_fwd_decode call: one decode query per sequence over the
    chunk-indexed long context (4 x 262,144 keys, 8 KV groups of 8 query heads, top-2048
    chunks of 64), the group's heads stacked.  HBM-bound: the selected K/V rows are read
    once per KV group.  The plain forward over the same plan is timed beside it."""
    import torch
    import block_sparse_attention_fwd_amd as bs
    from workloads.configs import make_chunk_gqa

    t0 = time.perf_counter()
    w = make_chunk_gqa("chunk-gqa-decode-b4-h64kv8-262144-d128", 5, B=4, Hq=64, Hkv=8, d=128, Nk=262144, Nq=1,
                       chunk=64, topk=2048, chunk_select=gpu_chunk_select)
    log(f"[bench] decode workload generated in {time.perf_counter() - t0:.1f} s")
    plan = bs.Plan.from_workload(w).upload()
    st = plan.stats

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    o = torch.empty((w.B, w.Nq, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    nws = bs.bsattn_decode_workspace_bytes(plan.handle)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    base = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), float(w.scale))

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, e0.elapsed_time(e1) / args.steps

    ms_dec, ev_dec = timed(lambda: bs.bsattn_fwd_decode(plan.handle, *base, ws.data_ptr(), nws, stream.cuda_stream))
    ms_fwd, ev_fwd = timed(lambda: bs.bsattn_fwd(plan.handle, *base, stream.cuda_stream))
    chunk, topk = int(w.k_offsets[1] - w.k_offsets[0]), int(w.sel_row_ptr[1] - w.sel_row_ptr[0])

    # the whole step on the device: chunk selection, page lists rebuilt from it, decode
    cp = bs.ChunkProblem()
    cp.B, cp.Hq, cp.Hkv, cp.Nq, cp.Nk, cp.d = w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d
    cp.chunk, cp.topk, cp.query_index, cp.reserved = chunk, topk, w.Nq - 1, 0
    cp.q_stride[:] = tuple(q.stride()[:3])
    cp.k_stride[:] = tuple(k.stride()[:3])
    summ = torch.empty((w.B, w.Hkv, -(-w.Nk // chunk), w.d), dtype=torch.float32, device=dev)
    chunks = torch.empty((w.B, w.Hkv, topk), dtype=torch.int32, device=dev)
    rp = torch.arange(0, w.B * w.Hkv * topk + 1, topk, dtype=torch.int32, device=dev)

    def pipeline():
        bs.bsattn_chunk_select(cp, q.data_ptr(), k.data_ptr(), summ.data_ptr(), chunks.data_ptr(), stream.cuda_stream)
        bs.bsattn_plan_update_selection(plan.handle, w.B, w.Hkv, rp.data_ptr(), chunks.data_ptr(), 0,
                                        stream.cuda_stream)
        bs.bsattn_fwd_decode(plan.handle, *base, ws.data_ptr(), nws, stream.cuda_stream)

    ms_pipe, _ = timed(pipeline)
    kv_bytes = w.B * w.Hkv * topk * chunk * w.d * 2 * 2   # selected K and V rows, once per KV group
    nbytes = kv_bytes + 2 * w.B * w.Nq * w.Hq * w.d * 2 + w.B * w.Hq * w.Nq * 4
    log(f"[bench] decode {ms_dec:.3f} ms (events {ev_dec:.3f}); plain forward over the same plan {ms_fwd:.3f} ms; "
        f"chunk selection + page lists on the device + decode {ms_pipe:.3f} ms")
    out = {
        "metric": "decode HBM GB/s (selected K/V read once per KV group), 1 GPU",
        "value": round(nbytes / (ms_dec * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_dec, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16 Q/K/V)",
        "config": {"workload": w.name, "pass": "decode", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq,
                   "Nk": w.Nk, "d": w.d, "chunk": chunk, "topk": topk, "useful_pairs": st["useful"],
                   "bytes": nbytes, "plain_forward_ms": round(ms_fwd, 4),
                   "speedup_over_plain_forward": round(ms_fwd / ms_dec, 2),
                   "device_step_ms": round(ms_pipe, 4)},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (ev_dec * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(nbytes / (ev_dec * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": measured_bytes("decode", DECODE_SRC, ("fwd_decode_kernel", "decode_merge_kernel")),
                     "kernel": "fwd_decode_kernel<128> + decode_merge_kernel<128>", "kernel_ms": round(ev_dec, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=None, help="benchmark workload 1-5 (default 3: video-DiT 3D)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-baseline sample budget (0 = skip)")
    ap.add_argument("--split-shapes", action="store_true",
                    help="launch the two tile shapes one after the other (timing each) instead of one launch")
    ap.add_argument("--natural-order", action="store_true",
                    help="dispatch Q tiles in Q-block order, ignoring the workload's locality hint")
    ap.add_argument("--fixed-tiles", action="store_true",
                    help="plan with the fixed-tile baseline (one 128x128 tile per selected block pair, no packing)")
    ap.add_argument("--decode", action="store_true",
                    help="time the head-stacked decode path on the chunk-indexed long context instead")
    ap.add_argument("--chunk-select", action="store_true",
                    help="time the chunk selection instead (default workload then 5: chunk-indexed GQA prefill)")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass instead (default workload then 4: independent Q/K partitions)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only run the dense-MFMA calibration (random and zero operands) and print its rates")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB, 5 times (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the forward pass would shard over (batch, head) with no exchange between GPUs).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_fwd_amd as bs
    from workloads.configs import make

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        a = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        c = torch.empty_like(a)
        for _ in range(5):
            c.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)
        return

    if args.mfma_probe:
        torch.cuda.set_device(0)
        res = {}
        for random in (True, False):
            tf, ghz, ms = bs.mfma_probe(iters=400000, random=random)
            res["random" if random else "zero"] = {"tflops": round(tf, 1), "ghz": round(ghz, 3), "ms": round(ms, 2)}
        print(json.dumps({"mfma_probe": res, "mfma": "v_mfma_f32_32x32x16_bf16",
                          "peak_tflops": PEAK_BF16_TFLOPS}), flush=True)
        return

    if args.workload is None:
        args.workload = 4 if args.bwd else (5 if args.chunk_select else 3)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.decode:
        bench_decode(args, dev)
        return
    t0 = time.perf_counter()
    w = make(args.workload, chunk_select=gpu_chunk_select)
    log(f"[bench] workload {w.name}: inputs generated in {time.perf_counter() - t0:.1f} s")

    if args.chunk_select:
        if args.workload != 5:
            raise SystemExit("--chunk-select runs on workload 5 (chunk-indexed GQA prefill)")
        bench_chunk_select(args, w, dev)
        return

    t0 = time.perf_counter()
    plan = bs.Plan.from_workload(w, block_order=not args.natural_order,
                                 flags=bs.PLAN_FIXED_TILES if args.fixed_tiles else 0)
    t_plan = time.perf_counter() - t0
    st = plan.stats
    plan.upload()
    log(f"[bench] plan built in {t_plan * 1e3:.1f} ms: {st}")
    if args.bwd:
        bench_bwd(args, w, plan, st, t_plan, dev)
        return

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    o = torch.empty((w.B, w.Nq, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    args_ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), float(w.scale), sh)
    split = args.split_shapes

    # HIP events on the launch stream: one step is one bsattn_fwd call (one kernel launch),
    # or with --split-shapes the 128x128 launch then the 64x256 launch
    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        if split:
            bs.bsattn_fwd_shape(plan.handle, bs.SHAPE_128x128, *args_ptrs)
            if evs is not None:
                evs[1].record(stream)
            bs.bsattn_fwd_shape(plan.handle, bs.SHAPE_64x256, *args_ptrs)
        else:
            bs.bsattn_fwd(plan.handle, *args_ptrs)
        if evs is not None:
            evs[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    t_all = np.array([e[0].elapsed_time(e[2]) for e in events])
    k_all = float(np.mean(t_all))
    flop = 4.0 * w.d * st["useful"]
    value = flop / (ms_step * 1e-3) / 1e12
    kernel_ms = {"launch": round(k_all, 4)}
    if split:
        t128 = np.array([e[0].elapsed_time(e[1]) for e in events])
        t64 = np.array([e[1].elapsed_time(e[2]) for e in events])
        kernel_ms = {"128x128": round(float(np.mean(t128)), 4), "64x256": round(float(np.mean(t64)), 4)}
        log(f"[bench] {ms_step:.3f} ms/step (wall); kernel 128x128 {kernel_ms['128x128']:.3f} ms, "
            f"kernel 64x256 {kernel_ms['64x256']:.3f} ms")
        # roofline of the dominant launch: the 128x128 tiles and their useful pairs
        k_dom, u_dom = kernel_ms["128x128"], st["useful_by_shape"][0]
        kname = f"fwd_kernel_pp<{w.d}, 128-row tiles>"
    else:
        log(f"[bench] {ms_step:.3f} ms/step (wall); one launch {k_all:.3f} ms (events)")
        k_dom, u_dom = k_all, st["useful"]
        kname = f"fwd_kernel_pp_fused<{w.d}> (128x128 and 64x256 tiles, one launch)"
    achieved = 4.0 * w.d * u_dom / (k_dom * 1e-3) / 1e12
    tag = "split" if split else "fused"
    traffic = measured_traffic(args.workload, tag)
    kv = measured_counters(args.workload)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": kname, "kernel_ms": round(k_dom, 4),
                "useful_pairs_per_launch": u_dom,
                # HBM rate of the counted bytes over this run's launch time, against 8 TB/s
                "hbm_GBps": round(traffic / (k_dom * 1e-3) / 1e9, 1) if traffic else None,
                "hbm_frac": round(traffic / (k_dom * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if traffic else None,
                # from the same counter runs (MFMA busy share of active SIMD cycles, LDS bank-conflict cycles)
                "mfma_busy_pct": float(kv[f"{tag}.mfma_busy_pct"]) if f"{tag}.mfma_busy_pct" in kv else None,
                "lds_bank_conflict_cycles": int(kv[f"{tag}.lds_bank_conflict_cycles"])
                if f"{tag}.lds_bank_conflict_cycles" in kv else None,
                "l2_hit_pct": float(kv[f"{tag}.l2_hit_pct"]) if f"{tag}.l2_hit_pct" in kv else None}

    # the rate the matrix cores sustain on this product alone, under the same power limit
    # (register operands of unit-normal-like spread, every SIMD busy; about half a second)
    probe_tf, probe_ghz, _ = bs.mfma_probe(iters=200000, random=True)
    roofline["mfma_probe_tflops"] = round(probe_tf, 1)
    roofline["mfma_probe_ghz"] = round(probe_ghz, 3)
    roofline["frac_of_mfma_probe"] = round(achieved / probe_tf, 4)
    log(f"[bench] dense-MFMA probe: {probe_tf:.1f} TFLOP/s at {probe_ghz:.3f} GHz; the launch reaches "
        f"{achieved / probe_tf:.3f} of it")

    cpu = None
    if args.cpu_seconds > 0:
        log(f"[bench] timing the CPU oracle for about {args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(w, args.cpu_seconds)

    out = {
        "metric": "useful-pair TFLOP/s (4*d*valid QK pairs/s), % bf16 MFMA peak, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V; block layout and selection as the workload defines)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "useful_pairs": st["useful"], "physical_pairs": st["physical"],
                   "physical_over_useful": round(st["physical"] / max(st["useful"], 1), 4),
                   "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
                   "launches": "per shape (--split-shapes)" if split else "one (both shapes)",
                   "kernel_ms": kernel_ms,
                   "step_ms_median_events": round(float(np.median(t_all)), 4),
                   "step_ms_min_events": round(float(np.min(t_all)), 4),
                   "plan": "fixed 128x128 tiles per selected block pair (no packing)" if args.fixed_tiles
                   else "packed pages, routed Q tiles",
                   "dispatch_order": "Q blocks in order" if (args.natural_order or w.q_block_order is None)
                   else "workload hint (cubes in slabs of two w columns, then t, h, w)",
                   "plan_ms": round(t_plan * 1e3, 2)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if args.fixed_tiles or args.natural_order:
        # the counter runs cover the default plan and order only
        for key in ("traffic", "hbm_GBps", "hbm_frac", "mfma_busy_pct", "lds_bank_conflict_cycles", "l2_hit_pct"):
            roofline[key] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
