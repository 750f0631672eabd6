"""Python binding of libbsattn: exact block-sparse softmax attention on MI355X.

Argument marshalling only.  Every step of the forward and backward passes -- planning
(host C++) and the attention itself (gfx950 HIP kernels) -- runs inside ``libbsattn.so``; PyTorch is
used here for device memory and streams.  The C entry points keep their C names
(``bsattn_plan_create``, ``bsattn_fwd``, ...); :class:`Plan` bundles them for tensors.

The library must have been built (``python -m block_sparse_attention_fwd_amd.build``);
any entry point called without it raises :class:`BsattnError` -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

__all__ = [
    "BsattnError", "Problem", "Layout", "Selection", "Stats", "PlanView", "Plan", "library",
    "bsattn_plan_create", "bsattn_plan_create_ex", "bsattn_plan_set_block_order", "PLAN_FIXED_TILES", "bsattn_plan_device_bytes", "bsattn_plan_upload", "bsattn_plan_stats",
    "bsattn_plan_export", "bsattn_plan_export_bwd", "PlanBwdView", "bsattn_fwd", "bsattn_fwd_shape",
    "bsattn_bwd_workspace_bytes", "bsattn_bwd", "bsattn_chunk_select", "ChunkProblem", "chunk_select",
    "bsattn_decode_workspace_bytes", "bsattn_fwd_decode", "bsattn_fwd_decode_noalloc", "bsattn_plan_update_selection",
    "bsattn_plan_destroy", "bsattn_status_string", "bsattn_last_hip_error", "SHAPE_128x128", "SHAPE_64x256", "PAGE_SIZE",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsattn.so")
DTYPE_BF16 = 1
SHAPE_128x128 = 0
SHAPE_64x256 = 1
PAGE_SIZE = 16
PLAN_FIXED_TILES = 1

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


class BsattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: status {status}"
        if _lib is not None:
            msg += f" ({_lib.bsattn_status_string(status).decode()})"
            if status == 6:
                msg += f", hipError {_lib.bsattn_last_hip_error()}"
        super().__init__(msg)


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("Nq", ctypes.c_int32), ("Nk", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32), ("q_pos0", ctypes.c_int64),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3)]


class Layout(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int32), ("offsets", _i32p), ("perm", _i32p)]


class Selection(ctypes.Structure):
    _fields_ = [("n_b", ctypes.c_int32), ("n_h", ctypes.c_int32), ("row_ptr", _i32p), ("kblk", _i32p)]


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("useful", "physical", "n_pages", "n_qtiles128", "n_qtiles64",
                                              "n_ktiles", "page_list_len", "n_units")] + [
        ("useful_by_shape", ctypes.c_int64 * 2), ("physical_by_shape", ctypes.c_int64 * 2)]


class PlanView(ctypes.Structure):
    _fields_ = [("n_pages", ctypes.c_int64), ("page_kblock", _i32p), ("page_slot0", _i32p),
                ("page_nvalid", _i32p), ("n_qtiles", ctypes.c_int64), ("qt_qblock", _i32p),
                ("qt_row0", _i32p), ("qt_rows", _i32p), ("qt_shape", _i32p), ("n_rows", ctypes.c_int64),
                ("pl_ptr", _i64p), ("pl_pages", _i32p)]


class ChunkProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("Nq", ctypes.c_int32),
                ("Nk", ctypes.c_int32), ("d", ctypes.c_int32), ("chunk", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("query_index", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3)]


class PlanBwdView(ctypes.Structure):
    _fields_ = [("n_qpages", ctypes.c_int64), ("qpage_qblock", _i32p), ("qpage_slot0", _i32p),
                ("qpage_nvalid", _i32p), ("n_dq_tiles", ctypes.c_int64), ("dqt_qblock", _i32p), ("dqt_row0", _i32p),
                ("dqt_rows", _i32p), ("n_kv_tiles", ctypes.c_int64), ("kvt_kblock", _i32p), ("kvt_row0", _i32p),
                ("kvt_rows", _i32p), ("n_trows", ctypes.c_int64), ("tpl_ptr", _i64p), ("tpl_pages", _i32p)]


_lib: Optional[ctypes.CDLL] = None

EXPORTED = ["bsattn_plan_create", "bsattn_plan_create_ex", "bsattn_plan_set_block_order", "bsattn_plan_device_bytes", "bsattn_plan_upload", "bsattn_plan_stats",
            "bsattn_plan_export", "bsattn_plan_export_bwd", "bsattn_fwd", "bsattn_fwd_shape",
            "bsattn_bwd_workspace_bytes", "bsattn_bwd", "bsattn_chunk_select", "bsattn_decode_workspace_bytes",
            "bsattn_fwd_decode", "bsattn_fwd_decode_noalloc", "bsattn_plan_update_selection", "bsattn_plan_destroy",
            "bsattn_mfma_probe", "bsattn_status_string",
            "bsattn_last_hip_error"]


def library() -> ctypes.CDLL:
    """Load libbsattn.so (once).  Raises BsattnError(-1) when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise BsattnError(-1, f"libbsattn.so not built at {LIB_PATH}; run python -m block_sparse_attention_fwd_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    lib.bsattn_plan_create.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Layout), ctypes.POINTER(Layout),
                                       ctypes.POINTER(Selection), ctypes.c_int32, ctypes.POINTER(vp)]
    lib.bsattn_plan_create_ex.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Layout), ctypes.POINTER(Layout),
                                          ctypes.POINTER(Selection), ctypes.c_int32, ctypes.c_int32,
                                          ctypes.POINTER(vp)]
    lib.bsattn_plan_set_block_order.argtypes = [vp, _i32p, ctypes.c_int32]
    lib.bsattn_plan_device_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    lib.bsattn_plan_upload.argtypes = [vp, vp, ctypes.c_size_t, vp]
    lib.bsattn_plan_stats.argtypes = [vp, ctypes.POINTER(Stats)]
    lib.bsattn_plan_export.argtypes = [vp, ctypes.POINTER(PlanView)]
    lib.bsattn_plan_export_bwd.argtypes = [vp, ctypes.POINTER(PlanBwdView)]
    lib.bsattn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp]
    lib.bsattn_fwd_shape.argtypes = [vp, ctypes.c_int32, vp, vp, vp, vp, vp, ctypes.c_float, vp]
    lib.bsattn_bwd_workspace_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    lib.bsattn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, ctypes.c_size_t, vp]
    lib.bsattn_decode_workspace_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    lib.bsattn_fwd_decode.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, ctypes.c_size_t, vp]
    lib.bsattn_fwd_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp]
    lib.bsattn_plan_update_selection.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp]
    lib.bsattn_chunk_select.argtypes = [ctypes.POINTER(ChunkProblem), vp, vp, vp, vp, vp]
    lib.bsattn_mfma_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.bsattn_plan_destroy.argtypes = [vp]
    lib.bsattn_status_string.argtypes = [ctypes.c_int]
    lib.bsattn_status_string.restype = ctypes.c_char_p
    lib.bsattn_last_hip_error.argtypes = []
    for n in EXPORTED:
        if n != "bsattn_status_string":
            getattr(lib, n).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise BsattnError(status, where)


# ---------------------------------------------------------------------------
# thin wrappers with the C names
# ---------------------------------------------------------------------------
def bsattn_plan_create(problem: Problem, q_layout: Layout, k_layout: Layout, selection: Selection,
                       page_size: int = PAGE_SIZE) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(library().bsattn_plan_create(ctypes.byref(problem), ctypes.byref(q_layout), ctypes.byref(k_layout),
                                        ctypes.byref(selection), page_size, ctypes.byref(h)), "bsattn_plan_create")
    return h


def bsattn_plan_create_ex(problem: Problem, q_layout: Layout, k_layout: Layout, selection: Selection,
                          page_size: int = PAGE_SIZE, flags: int = 0) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(library().bsattn_plan_create_ex(ctypes.byref(problem), ctypes.byref(q_layout), ctypes.byref(k_layout),
                                           ctypes.byref(selection), page_size, flags, ctypes.byref(h)),
           "bsattn_plan_create_ex")
    return h


def bsattn_plan_set_block_order(plan, order) -> None:
    o = np.ascontiguousarray(order, dtype=np.int32)
    _check(library().bsattn_plan_set_block_order(plan, o.ctypes.data_as(_i32p), int(o.shape[0])),
           "bsattn_plan_set_block_order")


def bsattn_plan_device_bytes(plan) -> int:
    n = ctypes.c_size_t()
    _check(library().bsattn_plan_device_bytes(plan, ctypes.byref(n)), "bsattn_plan_device_bytes")
    return int(n.value)


def bsattn_plan_upload(plan, dev_ptr: int, nbytes: int, stream: int = 0) -> None:
    _check(library().bsattn_plan_upload(plan, ctypes.c_void_p(dev_ptr), nbytes, ctypes.c_void_p(stream)),
           "bsattn_plan_upload")


def bsattn_plan_stats(plan) -> dict:
    s = Stats()
    _check(library().bsattn_plan_stats(plan, ctypes.byref(s)), "bsattn_plan_stats")
    out = {n: int(getattr(s, n)) for n, _ in Stats._fields_[:8]}
    out["useful_by_shape"] = [int(x) for x in s.useful_by_shape]
    out["physical_by_shape"] = [int(x) for x in s.physical_by_shape]
    return out


def bsattn_plan_export(plan) -> dict:
    v = PlanView()
    _check(library().bsattn_plan_export(plan, ctypes.byref(v)), "bsattn_plan_export")

    def arr(ptr, n, dt):
        if n == 0:
            return np.zeros(0, dtype=dt)
        return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dt, copy=True)

    n_pl = int(v.pl_ptr[v.n_rows]) if v.n_rows >= 0 else 0
    return {
        "page_kblock": arr(v.page_kblock, v.n_pages, np.int32), "page_slot0": arr(v.page_slot0, v.n_pages, np.int32),
        "page_nvalid": arr(v.page_nvalid, v.n_pages, np.int32), "qt_qblock": arr(v.qt_qblock, v.n_qtiles, np.int32),
        "qt_row0": arr(v.qt_row0, v.n_qtiles, np.int32), "qt_rows": arr(v.qt_rows, v.n_qtiles, np.int32),
        "qt_shape": arr(v.qt_shape, v.n_qtiles, np.int32), "pl_ptr": arr(v.pl_ptr, v.n_rows + 1, np.int64),
        "pl_pages": arr(v.pl_pages, n_pl, np.int32),
    }


def bsattn_plan_export_bwd(plan) -> dict:
    v = PlanBwdView()
    _check(library().bsattn_plan_export_bwd(plan, ctypes.byref(v)), "bsattn_plan_export_bwd")

    def arr(ptr, n, dt):
        if n == 0:
            return np.zeros(0, dtype=dt)
        return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dt, copy=True)

    n_tpl = int(v.tpl_ptr[v.n_trows]) if v.n_trows >= 0 else 0
    return {
        "qpage_qblock": arr(v.qpage_qblock, v.n_qpages, np.int32), "qpage_slot0": arr(v.qpage_slot0, v.n_qpages, np.int32),
        "qpage_nvalid": arr(v.qpage_nvalid, v.n_qpages, np.int32),
        "dqt_qblock": arr(v.dqt_qblock, v.n_dq_tiles, np.int32), "dqt_row0": arr(v.dqt_row0, v.n_dq_tiles, np.int32),
        "dqt_rows": arr(v.dqt_rows, v.n_dq_tiles, np.int32),
        "kvt_kblock": arr(v.kvt_kblock, v.n_kv_tiles, np.int32), "kvt_row0": arr(v.kvt_row0, v.n_kv_tiles, np.int32),
        "kvt_rows": arr(v.kvt_rows, v.n_kv_tiles, np.int32),
        "tpl_ptr": arr(v.tpl_ptr, v.n_trows + 1, np.int64), "tpl_pages": arr(v.tpl_pages, n_tpl, np.int32),
    }


def bsattn_fwd(plan, q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, scale: float,
               stream: int = 0) -> None:
    _check(library().bsattn_fwd(plan, ctypes.c_void_p(q_ptr), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
                                ctypes.c_void_p(o_ptr), ctypes.c_void_p(lse_ptr), ctypes.c_float(scale),
                                ctypes.c_void_p(stream)), "bsattn_fwd")


def bsattn_fwd_shape(plan, shape: int, q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
                     scale: float, stream: int = 0) -> None:
    _check(library().bsattn_fwd_shape(plan, shape, ctypes.c_void_p(q_ptr), ctypes.c_void_p(k_ptr),
                                      ctypes.c_void_p(v_ptr), ctypes.c_void_p(o_ptr), ctypes.c_void_p(lse_ptr),
                                      ctypes.c_float(scale), ctypes.c_void_p(stream)), "bsattn_fwd_shape")


def bsattn_bwd_workspace_bytes(plan) -> int:
    n = ctypes.c_size_t()
    _check(library().bsattn_bwd_workspace_bytes(plan, ctypes.byref(n)), "bsattn_bwd_workspace_bytes")
    return int(n.value)


def bsattn_bwd(plan, q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, do_ptr: int, dq_ptr: int,
               dk_ptr: int, dv_ptr: int, scale: float, ws_ptr: int, ws_bytes: int, stream: int = 0) -> None:
    vp = ctypes.c_void_p
    _check(library().bsattn_bwd(plan, vp(q_ptr), vp(k_ptr), vp(v_ptr), vp(o_ptr), vp(lse_ptr), vp(do_ptr),
                                vp(dq_ptr), vp(dk_ptr), vp(dv_ptr), ctypes.c_float(scale), vp(ws_ptr), ws_bytes,
                                vp(stream)), "bsattn_bwd")


def bsattn_decode_workspace_bytes(plan) -> int:
    n = ctypes.c_size_t()
    _check(library().bsattn_decode_workspace_bytes(plan, ctypes.byref(n)), "bsattn_decode_workspace_bytes")
    return int(n.value)


def bsattn_fwd_decode(plan, q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, scale: float, ws_ptr: int,
                      ws_bytes: int, stream: int = 0) -> None:
    vp = ctypes.c_void_p
    _check(library().bsattn_fwd_decode(plan, vp(q_ptr), vp(k_ptr), vp(v_ptr), vp(o_ptr), vp(lse_ptr),
                                       ctypes.c_float(scale), vp(ws_ptr), ws_bytes, vp(stream)), "bsattn_fwd_decode")


def bsattn_fwd_decode_noalloc(plan, q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, scale: float,
                              stream: int = 0) -> None:
    """bsattn_fwd_decode with the library's own device buffer for the partial states (no
    workspace argument, no allocation; calls overlapping on one GPU race)."""
    vp = ctypes.c_void_p
    _check(library().bsattn_fwd_decode_noalloc(plan, vp(q_ptr), vp(k_ptr), vp(v_ptr), vp(o_ptr), vp(lse_ptr),
                                               ctypes.c_float(scale), vp(stream)), "bsattn_fwd_decode_noalloc")


def bsattn_plan_update_selection(plan, n_b: int, n_h: int, row_ptr_ptr: int, kblk_ptr: int, status_ptr: int = 0,
                                 stream: int = 0) -> None:
    vp = ctypes.c_void_p
    _check(library().bsattn_plan_update_selection(plan, n_b, n_h, vp(row_ptr_ptr), vp(kblk_ptr),
                                                  vp(status_ptr) if status_ptr else None, vp(stream)),
           "bsattn_plan_update_selection")


def bsattn_chunk_select(problem: ChunkProblem, q_ptr: int, k_ptr: int, summ_ptr: int, chunks_ptr: int,
                        stream: int = 0) -> None:
    vp = ctypes.c_void_p
    _check(library().bsattn_chunk_select(ctypes.byref(problem), vp(q_ptr), vp(k_ptr), vp(summ_ptr), vp(chunks_ptr),
                                         vp(stream)), "bsattn_chunk_select")


def bsattn_mfma_probe(n_workgroups: int, iters: int, random: bool, clocks_ptr: int, stream: int = 0) -> None:
    vp = ctypes.c_void_p
    _check(library().bsattn_mfma_probe(n_workgroups, iters, 1 if random else 0, vp(clocks_ptr), vp(stream)),
           "bsattn_mfma_probe")


def mfma_probe(iters: int = 200000, random: bool = True, n_workgroups: int = 512, repeats: int = 2):
    """Sustained rate of the forward's MFMA on register operands alone (bsattn_mfma_probe):
    ``repeats`` launches back to back, the last one timed with HIP events on the current
    stream.  Returns (TFLOP/s, mean shader clock in GHz, launch ms)."""
    import torch
    clocks = torch.zeros(2 * n_workgroups, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for r in range(repeats):
        if r == repeats - 1:
            e0.record(stream)
        bsattn_mfma_probe(n_workgroups, iters, random, clocks.data_ptr(), stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    c = clocks.view(-1, 2).cpu().double()
    ghz = float(c[:, 0].sum() / (c[:, 1].sum() / 100e6)) / 1e9
    flop = float(n_workgroups) * 4 * iters * 32 * 32768.0
    return flop / (ms * 1e-3) / 1e12, ghz, ms


def chunk_select(q, k, Hkv: int, chunk: int, topk: int, query_index: int = -1, stream=None):
    """Chunk summaries and the top-k chunks per (batch, KV group) on the device.
    q [B, Nq, Hq, d], k [B, Nk, Hkv, d] bf16 device tensors (d contiguous).  Returns
    (summaries float32 [B, Hkv, n_chunks, d], chunks int32 [B, Hkv, topk] ascending)."""
    import torch
    B, Nq, Hq, d = q.shape
    Nk = k.shape[1]
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or q.stride(3) != 1 or k.stride(3) != 1:
        raise BsattnError(1, "chunk_select: q and k must be bf16 with d contiguous")
    pr = ChunkProblem()
    pr.B, pr.Hq, pr.Hkv, pr.Nq, pr.Nk, pr.d = B, Hq, Hkv, Nq, Nk, d
    pr.chunk, pr.topk = chunk, topk
    pr.query_index = query_index if query_index >= 0 else Nq + query_index
    pr.reserved = 0
    pr.q_stride[:] = tuple(q.stride()[:3])
    pr.k_stride[:] = tuple(k.stride()[:3])
    n = -(-Nk // chunk)
    summ = torch.empty((B, Hkv, n, d), dtype=torch.float32, device=q.device)
    chunks = torch.empty((B, Hkv, topk), dtype=torch.int32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    bsattn_chunk_select(pr, q.data_ptr(), k.data_ptr(), summ.data_ptr(), chunks.data_ptr(), stream)
    return summ, chunks


def bsattn_plan_destroy(plan) -> None:
    _check(library().bsattn_plan_destroy(plan), "bsattn_plan_destroy")


def bsattn_status_string(status: int) -> str:
    return library().bsattn_status_string(status).decode()


def bsattn_last_hip_error() -> int:
    return int(library().bsattn_last_hip_error())


# ---------------------------------------------------------------------------
# tensor-level convenience (marshalling only)
# ---------------------------------------------------------------------------
def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_i32p)


class Plan:
    """A plan for one problem: shape, strides, layouts and selection.

    Strides default to contiguous [B, N, H, d] tensors.  ``upload`` binds the plan's
    device tables to a caller-owned device buffer (a torch uint8 tensor is allocated
    when none is given); ``fwd`` runs the forward pass and ``bwd`` the backward pass on
    torch's current stream.
    """

    def __init__(self, B, Hq, Hkv, Nq, Nk, d, q_offsets, q_perm, k_offsets, k_perm, sel_nb, sel_nh, sel_row_ptr,
                 sel_kblk, causal=False, q_pos0=0, q_stride=None, k_stride=None, v_stride=None, o_stride=None,
                 page_size=PAGE_SIZE, flags=0):
        pr = Problem()
        pr.B, pr.Hq, pr.Hkv, pr.Nq, pr.Nk, pr.d = B, Hq, Hkv, Nq, Nk, d
        pr.dtype = DTYPE_BF16
        pr.causal = 1 if causal else 0
        pr.q_pos0 = int(q_pos0)
        def_q = (Nq * Hq * d, Hq * d, d)
        def_k = (Nk * Hkv * d, Hkv * d, d)
        for name, st, dflt in (("q_stride", q_stride, def_q), ("k_stride", k_stride, def_k),
                               ("v_stride", v_stride, def_k), ("o_stride", o_stride, def_q)):
            getattr(pr, name)[:] = tuple(int(x) for x in (st if st is not None else dflt))
        self.problem = pr
        self._keep = [_i32(q_offsets), _i32(q_perm), _i32(k_offsets), _i32(k_perm), _i32(sel_row_ptr),
                      _i32(sel_kblk)]
        qo, qp, ko, kp, rp, kb = self._keep
        ql = Layout(len(qo) - 1, _ptr(qo), _ptr(qp))
        kl = Layout(len(ko) - 1, _ptr(ko), _ptr(kp))
        sel = Selection(sel_nb, sel_nh, _ptr(rp), _ptr(kb) if kb is not None and kb.size else None)
        self.handle = bsattn_plan_create_ex(pr, ql, kl, sel, page_size, flags)
        self._keep = None
        self.device_buffer = None

    @classmethod
    def from_workload(cls, w, block_order=True, **kw):
        """A plan for a workload object; its Q-block dispatch hint (``q_block_order``) is
        applied unless ``block_order`` is False."""
        p = cls(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.q_offsets, w.q_perm, w.k_offsets, w.k_perm, w.sel_nb,
                w.sel_nh, w.sel_row_ptr, w.sel_kblk, causal=w.causal, q_pos0=w.q_pos0, **kw)
        order = getattr(w, "q_block_order", None)
        if block_order and order is not None:
            p.set_block_order(order)
        return p

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _lib is not None:
            _lib.bsattn_plan_destroy(h)
            self.handle = None

    @property
    def stats(self) -> dict:
        return bsattn_plan_stats(self.handle)

    def export(self) -> dict:
        return bsattn_plan_export(self.handle)

    def export_bwd(self) -> dict:
        return bsattn_plan_export_bwd(self.handle)

    def update_selection(self, n_b, n_h, row_ptr, kblk, status=None, stream=None):
        """Rebuild the page lists (the forward's and the backward's transposed ones) on the
        device from device int32 tensors (row_ptr, kblk); ``status`` (a device int32 tensor of
        one element) collects the error bits."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        for name, t in (("row_ptr", row_ptr), ("kblk", kblk)):
            if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
                raise BsattnError(1, f"update_selection: {name} must be a contiguous int32 device tensor")
        bsattn_plan_update_selection(self.handle, n_b, n_h, row_ptr.data_ptr(), kblk.data_ptr(),
                                     status.data_ptr() if status is not None else 0, stream)
        return self

    def set_block_order(self, order):
        """Dispatch order of the Q blocks (a locality hint; upload afterwards)."""
        bsattn_plan_set_block_order(self.handle, order)
        return self

    @property
    def device_bytes(self) -> int:
        return bsattn_plan_device_bytes(self.handle)

    def upload(self, buffer=None, stream=None):
        import torch
        n = self.device_bytes
        if buffer is None:
            buffer = torch.empty(n, dtype=torch.uint8, device="cuda")
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        bsattn_plan_upload(self.handle, buffer.data_ptr(), buffer.numel() * buffer.element_size(), stream)
        self.device_buffer = buffer
        return self

    def fwd(self, q, k, v, o=None, lse=None, scale=None, stream=None, shape=None):
        """Forward pass; ``shape`` (SHAPE_128x128 / SHAPE_64x256) restricts it to one tile shape."""
        import torch
        pr = self.problem
        if o is None:
            o = torch.empty((pr.B, pr.Nq, pr.Hq, pr.d), dtype=torch.bfloat16, device=q.device)
        if lse is None:
            lse = torch.empty((pr.B, pr.Hq, pr.Nq), dtype=torch.float32, device=q.device)
        for name, t, st in (("q", q, pr.q_stride), ("k", k, pr.k_stride), ("v", v, pr.v_stride),
                            ("o", o, pr.o_stride)):
            if t.dtype != torch.bfloat16 or not t.is_cuda:
                raise BsattnError(1, f"bsattn_fwd: {name} must be a bf16 device tensor")
            if tuple(t.stride()[:3]) != tuple(st) or t.stride(3) != 1:
                raise BsattnError(1, f"bsattn_fwd: {name} strides {t.stride()} differ from the plan's")
        if lse.dtype != torch.float32 or not lse.is_contiguous():
            raise BsattnError(1, "bsattn_fwd: lse must be contiguous float32 [B, Hq, Nq]")
        if scale is None:
            scale = 1.0 / float(pr.d) ** 0.5
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        if shape is None:
            bsattn_fwd(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), scale,
                       stream)
        else:
            bsattn_fwd_shape(self.handle, shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), scale, stream)
        return o, lse

    def bwd(self, q, k, v, o, lse, do, dq=None, dk=None, dv=None, workspace=None, scale=None, stream=None):
        """Backward pass: (dQ, dK, dV) for the upstream gradient ``do`` of O, given the
        forward's ``o`` and ``lse``.  Gradients take the strides of Q, K and V; dO O's."""
        import torch
        pr = self.problem
        if dq is None:
            dq = torch.empty_strided(q.shape, q.stride(), dtype=torch.bfloat16, device=q.device)
        if dk is None:
            dk = torch.empty_strided(k.shape, k.stride(), dtype=torch.bfloat16, device=k.device)
        if dv is None:
            dv = torch.empty_strided(v.shape, v.stride(), dtype=torch.bfloat16, device=v.device)
        for name, t, st in (("q", q, pr.q_stride), ("k", k, pr.k_stride), ("v", v, pr.v_stride),
                            ("o", o, pr.o_stride), ("do", do, pr.o_stride), ("dq", dq, pr.q_stride),
                            ("dk", dk, pr.k_stride), ("dv", dv, pr.v_stride)):
            if t.dtype != torch.bfloat16 or not t.is_cuda:
                raise BsattnError(1, f"bsattn_bwd: {name} must be a bf16 device tensor")
            if tuple(t.stride()[:3]) != tuple(st) or t.stride(3) != 1:
                raise BsattnError(1, f"bsattn_bwd: {name} strides {t.stride()} differ from the plan's")
        if lse.dtype != torch.float32 or not lse.is_contiguous():
            raise BsattnError(1, "bsattn_bwd: lse must be contiguous float32 [B, Hq, Nq]")
        nws = bsattn_bwd_workspace_bytes(self.handle)
        if workspace is None:
            workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
        if scale is None:
            scale = 1.0 / float(pr.d) ** 0.5
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        bsattn_bwd(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                   do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), scale, workspace.data_ptr(),
                   workspace.numel() * workspace.element_size(), stream)
        return dq, dk, dv

    def fwd_decode(self, q, k, v, o=None, lse=None, workspace=None, scale=None, stream=None):
        """The forward for small query blocks with the query heads of a KV group stacked
        (bsattn_fwd_decode); same outputs as ``fwd``."""
        import torch
        pr = self.problem
        if o is None:
            o = torch.empty((pr.B, pr.Nq, pr.Hq, pr.d), dtype=torch.bfloat16, device=q.device)
        if lse is None:
            lse = torch.empty((pr.B, pr.Hq, pr.Nq), dtype=torch.float32, device=q.device)
        for name, t, st in (("q", q, pr.q_stride), ("k", k, pr.k_stride), ("v", v, pr.v_stride),
                            ("o", o, pr.o_stride)):
            if t.dtype != torch.bfloat16 or not t.is_cuda:
                raise BsattnError(1, f"bsattn_fwd_decode: {name} must be a bf16 device tensor")
            if tuple(t.stride()[:3]) != tuple(st) or t.stride(3) != 1:
                raise BsattnError(1, f"bsattn_fwd_decode: {name} strides {t.stride()} differ from the plan's")
        nws = bsattn_decode_workspace_bytes(self.handle)
        if workspace is None:
            workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
        if scale is None:
            scale = 1.0 / float(pr.d) ** 0.5
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        bsattn_fwd_decode(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), scale,
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream)
        return o, lse
