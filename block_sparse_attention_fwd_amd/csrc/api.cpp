// C-ABI entry points of libbsattn (declared in include/bsattn.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <new>

#include "bsattn.h"
#include "kernel_params.hpp"
#include "plan.hpp"

namespace bsattn {
hipError_t launch_fwd_shape(const FwdParams& p, int shape, int d, hipStream_t stream);
hipError_t launch_fwd(const FwdParams& p, int d, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, int d, hipStream_t stream);
hipError_t launch_chunk_select(const ChunkParams& p, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t stream);
hipError_t launch_plan_update(const PlanUpdateParams& p, hipStream_t stream);
hipError_t launch_mfma_probe(int n_workgroups, int iters, int random, uint64_t* clocks, hipStream_t stream);
hipError_t decode_scratch(void** ptr, size_t* bytes);
}

namespace {
thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = int(e);
  return BSATTN_E_HIP;
}
}  // namespace

extern "C" {

int bsattn_plan_create_ex(const bsattn_problem* problem, const bsattn_layout* q_layout,
                          const bsattn_layout* k_layout, const bsattn_selection* selection,
                          int32_t page_size, int32_t flags, bsattn_plan** out) {
  if (out == nullptr) return BSATTN_E_ARG;
  *out = nullptr;
  if (problem == nullptr || q_layout == nullptr || k_layout == nullptr || selection == nullptr)
    return BSATTN_E_ARG;
  if (page_size != bsattn::kPage) return BSATTN_E_UNSUPPORTED;
  bsattn_plan* p = new (std::nothrow) bsattn_plan();
  if (p == nullptr) return BSATTN_E_OOM;
  int st;
  try {
    st = bsattn::build_plan(*problem, *q_layout, *k_layout, *selection, flags, p);
  } catch (const std::bad_alloc&) {
    st = BSATTN_E_OOM;
  } catch (...) {
    st = BSATTN_E_ARG;
  }
  if (st != BSATTN_OK) {
    delete p;
    return st;
  }
  *out = p;
  return BSATTN_OK;
}

int bsattn_plan_create(const bsattn_problem* problem, const bsattn_layout* q_layout,
                       const bsattn_layout* k_layout, const bsattn_selection* selection,
                       int32_t page_size, bsattn_plan** out) {
  return bsattn_plan_create_ex(problem, q_layout, k_layout, selection, page_size, 0, out);
}

int bsattn_plan_set_block_order(bsattn_plan* plan, const int32_t* order, int32_t n_qblocks) {
  if (plan == nullptr) return BSATTN_E_ARG;
  try {
    return bsattn::set_block_order(plan, order, n_qblocks);
  } catch (const std::bad_alloc&) {
    return BSATTN_E_OOM;
  }
}

int bsattn_plan_device_bytes(const bsattn_plan* plan, size_t* bytes) {
  if (plan == nullptr || bytes == nullptr) return BSATTN_E_ARG;
  *bytes = plan->image.size();
  return BSATTN_OK;
}

int bsattn_plan_upload(bsattn_plan* plan, void* dev, size_t bytes, void* stream) {
  if (plan == nullptr || dev == nullptr) return BSATTN_E_ARG;
  if (bytes < plan->image.size() || (reinterpret_cast<uintptr_t>(dev) & 255) != 0) return BSATTN_E_ARG;
  hipError_t e = hipMemcpyAsync(dev, plan->image.data(), plan->image.size(), hipMemcpyHostToDevice,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  plan->dev = dev;
  return BSATTN_OK;
}

int bsattn_plan_update_selection(bsattn_plan* plan, int32_t n_b, int32_t n_h, const int32_t* row_ptr,
                                 const int32_t* kblk, int32_t* status, void* stream) {
  if (plan == nullptr || row_ptr == nullptr) return BSATTN_E_ARG;
  if (plan->dev == nullptr) return BSATTN_E_STATE;
  if (n_b != plan->sel_nb || n_h != plan->sel_nh) return BSATTN_E_ARG;
  if (plan->flags != 0) return BSATTN_E_UNSUPPORTED;
  uint8_t* base = static_cast<uint8_t*>(plan->dev);
  bsattn::PlanUpdateParams up{};
  up.row_ptr = row_ptr;
  up.kblk = kblk;
  up.first_page = reinterpret_cast<const int32_t*>(base + plan->off_firstpage);
  up.page_ent = reinterpret_cast<const int32_t*>(base + plan->off_pageent);
  up.pl_ptr = reinterpret_cast<int32_t*>(base + plan->off_plptr);
  up.pl_ent = reinterpret_cast<int32_t*>(base + plan->off_plent);
  up.status = status;
  up.n_rows = int32_t(plan->pl_ptr.size()) - 1;
  up.nkb = plan->nkb;
  up.capacity = int32_t(plan->ent_capacity);
  up.first_qpage = reinterpret_cast<const int32_t*>(base + plan->off_firstqpage);
  up.qpage_ent = reinterpret_cast<const int32_t*>(base + plan->off_qpageent);
  up.tpl_ptr = reinterpret_cast<int32_t*>(base + plan->off_tplptr);
  up.tpl_ent = reinterpret_cast<int32_t*>(base + plan->off_tplent);
  up.n_units = plan->n_units;
  up.nqb = plan->nqb;
  up.tcapacity = int32_t(plan->tent_capacity);
  hipError_t e = bsattn::launch_plan_update(up, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return BSATTN_OK;
}

int bsattn_plan_stats(const bsattn_plan* plan, bsattn_stats* stats) {
  if (plan == nullptr || stats == nullptr) return BSATTN_E_ARG;
  *stats = plan->stats;
  return BSATTN_OK;
}

int bsattn_plan_export(const bsattn_plan* plan, bsattn_plan_view* v) {
  if (plan == nullptr || v == nullptr) return BSATTN_E_ARG;
  v->n_pages = int64_t(plan->page_kblock.size());
  v->page_kblock = plan->page_kblock.data();
  v->page_slot0 = plan->page_slot0.data();
  v->page_nvalid = plan->page_nvalid.data();
  v->n_qtiles = int64_t(plan->qt_qblock.size());
  v->qt_qblock = plan->qt_qblock.data();
  v->qt_row0 = plan->qt_row0.data();
  v->qt_rows = plan->qt_rows.data();
  v->qt_shape = plan->qt_shape.data();
  v->n_rows = int64_t(plan->pl_ptr.size()) - 1;
  v->pl_ptr = plan->pl_ptr.data();
  v->pl_pages = plan->pl_pages.data();
  return BSATTN_OK;
}

int bsattn_plan_export_bwd(const bsattn_plan* plan, bsattn_plan_bwd_view* v) {
  if (plan == nullptr || v == nullptr) return BSATTN_E_ARG;
  v->n_qpages = int64_t(plan->qpage_qblock.size());
  v->qpage_qblock = plan->qpage_qblock.data();
  v->qpage_slot0 = plan->qpage_slot0.data();
  v->qpage_nvalid = plan->qpage_nvalid.data();
  v->n_dq_tiles = int64_t(plan->dqt_row0.size());
  v->dqt_qblock = plan->dqt_qblock.data();
  v->dqt_row0 = plan->dqt_row0.data();
  v->dqt_rows = plan->dqt_rows.data();
  v->n_kv_tiles = int64_t(plan->kvt_row0.size());
  v->kvt_kblock = plan->kvt_kblock.data();
  v->kvt_row0 = plan->kvt_row0.data();
  v->kvt_rows = plan->kvt_rows.data();
  v->n_trows = int64_t(plan->tpl_ptr.size()) - 1;
  v->tpl_ptr = plan->tpl_ptr.data();
  v->tpl_pages = plan->tpl_pages.data();
  return BSATTN_OK;
}

}  // extern "C"

namespace {
// Validates the arguments and launches the kernels of the shapes in [sh0, sh1).
int run_fwd(const bsattn_plan* plan, int sh0, int sh1, const void* q, const void* k, const void* v, void* o,
            float* lse, float scale, void* stream) {
  if (plan == nullptr) return BSATTN_E_ARG;
  if (plan->dev == nullptr) return BSATTN_E_STATE;
  const bsattn_problem& pr = plan->prob;
  if (pr.Nq == 0) return BSATTN_OK;
  if (q == nullptr || o == nullptr || lse == nullptr) return BSATTN_E_ARG;
  if (pr.Nk > 0 && (k == nullptr || v == nullptr)) return BSATTN_E_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return BSATTN_E_ARG;
  // every row must start on a 16-byte boundary: aligned bases and strides in multiples of 8
  auto aligned = [](const void* ptr, const int64_t* st) {
    return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0 && st[0] % 8 == 0 && st[1] % 8 == 0 && st[2] % 8 == 0;
  };
  if (!aligned(q, pr.q_stride) || !aligned(o, pr.o_stride)) return BSATTN_E_ARG;
  if (pr.Nk > 0 && (!aligned(k, pr.k_stride) || !aligned(v, pr.v_stride))) return BSATTN_E_ARG;
  for (const int64_t* st : {pr.q_stride, pr.k_stride, pr.v_stride, pr.o_stride})
    if (st[0] < 0 || st[1] < 0 || st[2] < 0) return BSATTN_E_ARG;
  // K/V rows of one (batch, KV head) are addressed with 32-bit byte offsets
  const int64_t k_extent = pr.Nk > 0 ? (int64_t(pr.Nk) - 1) * pr.k_stride[1] * 2 + pr.d * 2 : 0;
  const int64_t v_extent = pr.Nk > 0 ? (int64_t(pr.Nk) - 1) * pr.v_stride[1] * 2 + pr.d * 2 : 0;
  if (k_extent > 0xffffffffLL || v_extent > 0xffffffffLL) return BSATTN_E_UNSUPPORTED;

  const uint8_t* base = static_cast<const uint8_t*>(plan->dev);
  bsattn::FwdParams fp{};
  fp.q = q; fp.k = k; fp.v = v; fp.o = o; fp.lse = lse;
  fp.q_sb = pr.q_stride[0]; fp.q_sn = pr.q_stride[1]; fp.q_sh = pr.q_stride[2];
  fp.k_sb = pr.k_stride[0]; fp.k_sn = pr.k_stride[1]; fp.k_sh = pr.k_stride[2];
  fp.v_sb = pr.v_stride[0]; fp.v_sn = pr.v_stride[1]; fp.v_sh = pr.v_stride[2];
  fp.o_sb = pr.o_stride[0]; fp.o_sn = pr.o_stride[1]; fp.o_sh = pr.o_stride[2];
  fp.pl_ptr = reinterpret_cast<const int32_t*>(base + plan->off_plptr);
  fp.pl_ent = reinterpret_cast<const int32_t*>(base + plan->off_plent);
  fp.qperm = plan->has_qperm ? reinterpret_cast<const int32_t*>(base + plan->off_qperm) : nullptr;
  fp.kperm = plan->has_kperm ? reinterpret_cast<const int32_t*>(base + plan->off_kperm) : nullptr;
  fp.q_pos0 = pr.q_pos0;
  fp.k_extent = uint32_t(k_extent);
  fp.v_extent = uint32_t(v_extent);
  fp.k_sn_bytes = uint32_t(pr.k_stride[1] * 2);
  fp.v_sn_bytes = uint32_t(pr.v_stride[1] * 2);
  fp.B = pr.B; fp.Hq = pr.Hq; fp.Hkv = pr.Hkv; fp.Nq = pr.Nq; fp.Nk = pr.Nk;
  fp.grp = pr.Hq / pr.Hkv;
  fp.nqb = plan->nqb;
  fp.sel_nh = plan->sel_nh;
  fp.ub_mul = (plan->sel_nb == pr.B) ? 1 : 0;
  fp.uh_div = (plan->sel_nh == pr.Hq) ? 1 : (plan->sel_nh == pr.Hkv ? fp.grp : pr.Hq);
  fp.causal = pr.causal;
  fp.scale = scale;
  fp.scale_log2 = scale * 1.4426950408889634f;

  const int64_t bh = int64_t(pr.B) * pr.Hq;
  for (int sh = sh0; sh < sh1; ++sh) {
    const int64_t nw = int64_t(plan->n_qt[sh]) * bh;
    if (nw >= (int64_t(1) << 31)) return BSATTN_E_UNSUPPORTED;
  }
  if (int64_t(plan->n_qt[0]) * bh + int64_t(plan->n_qt[1]) * bh >= (int64_t(1) << 31)) return BSATTN_E_UNSUPPORTED;
  if (sh0 == 0 && sh1 == bsattn::kShapes) {
    // both shapes: one launch where the kernels allow it
    fp.qtiles = reinterpret_cast<const bsattn::QTileDev*>(base + plan->off_qt[0]);
    fp.n_qtiles = plan->n_qt[0];
    fp.n_work = int32_t(int64_t(plan->n_qt[0]) * bh);
    fp.qtiles2 = reinterpret_cast<const bsattn::QTileDev*>(base + plan->off_qt[1]);
    fp.n_qtiles2 = plan->n_qt[1];
    fp.n_work2 = int32_t(int64_t(plan->n_qt[1]) * bh);
    hipError_t e = bsattn::launch_fwd(fp, pr.d, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e);
    return BSATTN_OK;
  }
  for (int sh = sh0; sh < sh1; ++sh) {
    bsattn::FwdParams f = fp;
    f.qtiles = reinterpret_cast<const bsattn::QTileDev*>(base + plan->off_qt[sh]);
    f.n_qtiles = plan->n_qt[sh];
    f.n_work = int32_t(int64_t(plan->n_qt[sh]) * bh);
    hipError_t e = bsattn::launch_fwd_shape(f, sh, pr.d, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e);
  }
  return BSATTN_OK;
}
}  // namespace

namespace {
size_t bwd_workspace_bytes(const bsattn_problem& pr) {
  const size_t n = size_t(pr.B) * size_t(pr.Hq) * size_t(pr.Nq) * sizeof(float);
  return std::max<size_t>((n + 255) & ~size_t(255), 256);
}

// Validates the arguments and launches D = rowsum(dO * O), then dK/dV and dQ.
int run_bwd(const bsattn_plan* plan, const void* q, const void* k, const void* v, const void* o, const float* lse,
            const void* dout, void* dq, void* dk, void* dv, float scale, void* workspace, size_t workspace_bytes,
            void* stream) {
  if (plan == nullptr) return BSATTN_E_ARG;
  if (plan->dev == nullptr) return BSATTN_E_STATE;
  const bsattn_problem& pr = plan->prob;
  if (!std::isfinite(scale) || !(scale > 0.f)) return BSATTN_E_ARG;
  if (workspace == nullptr || workspace_bytes < bwd_workspace_bytes(pr) ||
      (reinterpret_cast<uintptr_t>(workspace) & 15) != 0)
    return BSATTN_E_ARG;
  auto aligned = [](const void* ptr, const int64_t* st) {
    return ptr != nullptr && (reinterpret_cast<uintptr_t>(ptr) & 15) == 0 && st[0] % 8 == 0 && st[1] % 8 == 0 &&
           st[2] % 8 == 0 && st[0] >= 0 && st[1] >= 0 && st[2] >= 0;
  };
  if (pr.Nq > 0 && (!aligned(q, pr.q_stride) || !aligned(dq, pr.q_stride) || !aligned(o, pr.o_stride) ||
                    !aligned(dout, pr.o_stride) || lse == nullptr))
    return BSATTN_E_ARG;
  if (pr.Nk > 0 && (!aligned(k, pr.k_stride) || !aligned(dk, pr.k_stride) || !aligned(v, pr.v_stride) ||
                    !aligned(dv, pr.v_stride)))
    return BSATTN_E_ARG;
  // rows of one (batch, head) slice are addressed with 32-bit byte offsets
  auto extent = [&](int32_t n, const int64_t* st) { return n > 0 ? (int64_t(n) - 1) * st[1] * 2 + pr.d * 2 : 0; };
  const int64_t ext[4] = {extent(pr.Nq, pr.q_stride), extent(pr.Nq, pr.o_stride), extent(pr.Nk, pr.k_stride),
                          extent(pr.Nk, pr.v_stride)};
  for (int64_t e : ext)
    if (e > 0xffffffffLL) return BSATTN_E_UNSUPPORTED;
  const int64_t n_dq = int64_t(pr.B) * pr.Hq * int64_t(plan->dqt_row0.size());
  const int64_t n_kv = int64_t(pr.B) * pr.Hkv * int64_t(plan->kvt_row0.size());
  if (n_dq >= (int64_t(1) << 31) || n_kv >= (int64_t(1) << 31)) return BSATTN_E_UNSUPPORTED;
  // the dK/dV kernel reads the transposed page entries through 32-bit byte offsets
  if (plan->tpl_pages.size() + bsattn::kEntryPad >= (size_t(1) << 29)) return BSATTN_E_UNSUPPORTED;

  const uint8_t* base = static_cast<const uint8_t*>(plan->dev);
  bsattn::BwdParams bp{};
  bp.q = q; bp.k = k; bp.v = v; bp.o = o; bp.dout = dout; bp.lse = lse;
  bp.dq = dq; bp.dk = dk; bp.dv = dv; bp.dvec = static_cast<float*>(workspace);
  bp.q_sb = pr.q_stride[0]; bp.q_sn = pr.q_stride[1]; bp.q_sh = pr.q_stride[2];
  bp.k_sb = pr.k_stride[0]; bp.k_sn = pr.k_stride[1]; bp.k_sh = pr.k_stride[2];
  bp.v_sb = pr.v_stride[0]; bp.v_sn = pr.v_stride[1]; bp.v_sh = pr.v_stride[2];
  bp.o_sb = pr.o_stride[0]; bp.o_sn = pr.o_stride[1]; bp.o_sh = pr.o_stride[2];
  bp.dq_tiles = reinterpret_cast<const bsattn::QTileDev*>(base + plan->off_dqt);
  bp.kv_tiles = reinterpret_cast<const bsattn::QTileDev*>(base + plan->off_kvt);
  bp.pl_ptr = reinterpret_cast<const int32_t*>(base + plan->off_plptr);
  bp.pl_ent = reinterpret_cast<const int32_t*>(base + plan->off_plent);
  bp.tpl_ptr = reinterpret_cast<const int32_t*>(base + plan->off_tplptr);
  bp.tpl_ent = reinterpret_cast<const int32_t*>(base + plan->off_tplent);
  bp.qperm = plan->has_qperm ? reinterpret_cast<const int32_t*>(base + plan->off_qperm) : nullptr;
  bp.kperm = plan->has_kperm ? reinterpret_cast<const int32_t*>(base + plan->off_kperm) : nullptr;
  bp.q_pos0 = pr.q_pos0;
  bp.q_extent = uint32_t(ext[0]); bp.o_extent = uint32_t(ext[1]);
  bp.k_extent = uint32_t(ext[2]); bp.v_extent = uint32_t(ext[3]);
  bp.q_sn_bytes = uint32_t(pr.q_stride[1] * 2); bp.o_sn_bytes = uint32_t(pr.o_stride[1] * 2);
  bp.k_sn_bytes = uint32_t(pr.k_stride[1] * 2); bp.v_sn_bytes = uint32_t(pr.v_stride[1] * 2);
  bp.n_dq_tiles = int32_t(plan->dqt_row0.size());
  bp.n_dq_split = plan->n_dqt_split;
  bp.n_kv_tiles = int32_t(plan->kvt_row0.size());
  bp.B = pr.B; bp.Hq = pr.Hq; bp.Hkv = pr.Hkv; bp.Nq = pr.Nq; bp.Nk = pr.Nk;
  bp.grp = pr.Hq / pr.Hkv;
  bp.nqb = plan->nqb;
  bp.nkb = plan->nkb;
  bp.sel_nh = plan->sel_nh;
  bp.ub_mul = (plan->sel_nb == pr.B) ? 1 : 0;
  bp.uh_div = (plan->sel_nh == pr.Hq) ? 1 : (plan->sel_nh == pr.Hkv ? bp.grp : pr.Hq);
  bp.causal = pr.causal;
  bp.scale = scale;
  bp.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = bsattn::launch_bwd(bp, pr.d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return BSATTN_OK;
}
}  // namespace

extern "C" {

namespace {
// Split of the decode work: every Q block fits one stacked tile (n * group <= 32, so every
// tile is a 64-row tile), the query heads of a group share a selection unit, and each page
// list is cut into n_splits ranges of pps pages (a multiple of 8) so that about 512
// workgroups run: the walk keeps two workgroups on each of the 256 CUs, so the whole launch
// is one round (one start-up per slot, no tail; 2048 or 4096 smaller splits measured 2-7 %
// slower).  Returns BSATTN_OK or BSATTN_E_UNSUPPORTED.
int decode_geometry(const bsattn_plan* plan, int32_t* n_splits, int32_t* pps, size_t* ws_bytes) {
  const bsattn_problem& pr = plan->prob;
  const int32_t grp = pr.Hq / pr.Hkv;
  if (plan->flags != 0 || plan->n_qt[0] != 0) return BSATTN_E_UNSUPPORTED;
  if (plan->sel_nh == pr.Hq && grp > 1) return BSATTN_E_UNSUPPORTED;
  int32_t max_rows = 0;
  for (size_t t = 0; t < plan->qt_rows.size(); ++t) max_rows = std::max(max_rows, plan->qt_rows[t]);
  if (int64_t(max_rows) * grp > 32) return BSATTN_E_UNSUPPORTED;
  int64_t max_list = 0;
  for (size_t r = 0; r + 1 < plan->pl_ptr.size(); ++r) max_list = std::max(max_list, plan->pl_ptr[r + 1] - plan->pl_ptr[r]);
  const int64_t items = int64_t(pr.B) * pr.Hkv * plan->n_qt[1];
  int64_t ns = items > 0 ? (512 + items - 1) / items : 1;
  ns = std::max<int64_t>(1, std::min<int64_t>({ns, (max_list + 7) / 8, int64_t(256)}));
  int64_t per = (max_list + ns - 1) / ns;
  per = std::max<int64_t>(8, (per + 7) / 8 * 8);
  ns = std::max<int64_t>(1, (max_list + per - 1) / per);
  if (items * ns >= (int64_t(1) << 31) || per >= (int64_t(1) << 30)) return BSATTN_E_UNSUPPORTED;
  *n_splits = int32_t(ns);
  *pps = int32_t(per);
  *ws_bytes = std::max<size_t>(256, size_t(items * ns) * 32 * size_t(pr.d + 2) * sizeof(float));
  return BSATTN_OK;
}
}  // namespace

int bsattn_decode_workspace_bytes(const bsattn_plan* plan, size_t* bytes) {
  if (plan == nullptr || bytes == nullptr) return BSATTN_E_ARG;
  int32_t ns, per;
  return decode_geometry(plan, &ns, &per, bytes);
}

int bsattn_fwd_decode(const bsattn_plan* plan, const void* q, const void* k, const void* v, void* o, float* lse,
                      float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (plan == nullptr) return BSATTN_E_ARG;
  if (plan->dev == nullptr) return BSATTN_E_STATE;
  const bsattn_problem& pr = plan->prob;
  int32_t ns = 0, per = 0;
  size_t need = 0;
  const int st = decode_geometry(plan, &ns, &per, &need);
  if (st != BSATTN_OK) return st;
  if (pr.Nq == 0) return BSATTN_OK;
  if (q == nullptr || o == nullptr || lse == nullptr || workspace == nullptr || workspace_bytes < need) return BSATTN_E_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0) return BSATTN_E_ARG;
  if (pr.Nk > 0 && (k == nullptr || v == nullptr)) return BSATTN_E_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return BSATTN_E_ARG;
  auto aligned = [](const void* ptr, const int64_t* sd) {
    return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0 && sd[0] % 8 == 0 && sd[1] % 8 == 0 && sd[2] % 8 == 0 &&
           sd[0] >= 0 && sd[1] >= 0 && sd[2] >= 0;
  };
  if (!aligned(q, pr.q_stride) || !aligned(o, pr.o_stride)) return BSATTN_E_ARG;
  if (pr.Nk > 0 && (!aligned(k, pr.k_stride) || !aligned(v, pr.v_stride))) return BSATTN_E_ARG;
  const int64_t k_extent = pr.Nk > 0 ? (int64_t(pr.Nk) - 1) * pr.k_stride[1] * 2 + pr.d * 2 : 0;
  const int64_t v_extent = pr.Nk > 0 ? (int64_t(pr.Nk) - 1) * pr.v_stride[1] * 2 + pr.d * 2 : 0;
  if (k_extent > 0xffffffffLL || v_extent > 0xffffffffLL) return BSATTN_E_UNSUPPORTED;
  const uint8_t* base = static_cast<const uint8_t*>(plan->dev);
  bsattn::DecodeParams dp{};
  dp.q = q; dp.k = k; dp.v = v; dp.o = o; dp.lse = lse;
  dp.q_sb = pr.q_stride[0]; dp.q_sn = pr.q_stride[1]; dp.q_sh = pr.q_stride[2];
  dp.k_sb = pr.k_stride[0]; dp.k_sn = pr.k_stride[1]; dp.k_sh = pr.k_stride[2];
  dp.v_sb = pr.v_stride[0]; dp.v_sn = pr.v_stride[1]; dp.v_sh = pr.v_stride[2];
  dp.o_sb = pr.o_stride[0]; dp.o_sn = pr.o_stride[1]; dp.o_sh = pr.o_stride[2];
  dp.qtiles = reinterpret_cast<const bsattn::QTileDev*>(base + plan->off_qt[1]);
  dp.pl_ptr = reinterpret_cast<const int32_t*>(base + plan->off_plptr);
  dp.pl_ent = reinterpret_cast<const int32_t*>(base + plan->off_plent);
  dp.qperm = plan->has_qperm ? reinterpret_cast<const int32_t*>(base + plan->off_qperm) : nullptr;
  dp.kperm = plan->has_kperm ? reinterpret_cast<const int32_t*>(base + plan->off_kperm) : nullptr;
  dp.opart = static_cast<float*>(workspace);
  const int64_t items = int64_t(pr.B) * pr.Hkv * plan->n_qt[1];
  dp.mlpart = dp.opart + size_t(items * ns) * 32 * size_t(pr.d);
  dp.q_pos0 = pr.q_pos0;
  dp.k_extent = uint32_t(k_extent);
  dp.v_extent = uint32_t(v_extent);
  dp.k_sn_bytes = uint32_t(pr.k_stride[1] * 2);
  dp.v_sn_bytes = uint32_t(pr.v_stride[1] * 2);
  dp.n_qtiles = plan->n_qt[1];
  dp.n_splits = ns;
  dp.pps = per;
  dp.B = pr.B; dp.Hq = pr.Hq; dp.Hkv = pr.Hkv; dp.Nq = pr.Nq; dp.Nk = pr.Nk;
  dp.grp = pr.Hq / pr.Hkv;
  dp.nqb = plan->nqb;
  dp.sel_nh = plan->sel_nh;
  dp.ub_mul = (plan->sel_nb == pr.B) ? 1 : 0;
  dp.uh_div = (plan->sel_nh == pr.Hq) ? 1 : (plan->sel_nh == pr.Hkv ? dp.grp : pr.Hq);
  dp.causal = pr.causal;
  dp.scale = scale;
  dp.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = bsattn::launch_decode(dp, pr.d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return BSATTN_OK;
}

int bsattn_fwd_decode_noalloc(const bsattn_plan* plan, const void* q, const void* k, const void* v, void* o,
                              float* lse, float scale, void* stream) {
  if (plan == nullptr) return BSATTN_E_ARG;
  int32_t ns = 0, per = 0;
  size_t need = 0;
  const int st = decode_geometry(plan, &ns, &per, &need);
  if (st != BSATTN_OK) return st;
  if (need > bsattn::kDecodeScratchBytes) return BSATTN_E_UNSUPPORTED;
  if (plan->dev == nullptr) return BSATTN_E_STATE;
  void* ws = nullptr;
  size_t bytes = 0;
  const hipError_t e = bsattn::decode_scratch(&ws, &bytes);
  if (e != hipSuccess) return hip_fail(e);
  return bsattn_fwd_decode(plan, q, k, v, o, lse, scale, ws, bytes, stream);
}

int bsattn_chunk_select(const bsattn_chunk_problem* pr, const void* q, const void* k, float* summaries,
                        int32_t* chunks, void* stream) {
  if (pr == nullptr || q == nullptr || k == nullptr || summaries == nullptr || chunks == nullptr) return BSATTN_E_ARG;
  if (pr->B < 1 || pr->Hq < 1 || pr->Hkv < 1 || pr->Hq % pr->Hkv != 0 || pr->Nq < 1 || pr->Nk < 1 || pr->chunk < 1)
    return BSATTN_E_ARG;
  if (pr->query_index < 0 || pr->query_index >= pr->Nq) return BSATTN_E_ARG;
  if (pr->d != 64 && pr->d != 128) return BSATTN_E_UNSUPPORTED;
  const int64_t n = (int64_t(pr->Nk) + pr->chunk - 1) / pr->chunk;
  if (pr->topk < 1 || pr->topk > n) return BSATTN_E_ARG;
  if (n > 8192) return BSATTN_E_UNSUPPORTED;
  for (const int64_t* st : {pr->q_stride, pr->k_stride})
    if (st[0] < 0 || st[1] < 0 || st[2] < 0 || st[0] % 8 != 0 || st[1] % 8 != 0 || st[2] % 8 != 0) return BSATTN_E_ARG;
  if ((reinterpret_cast<uintptr_t>(k) & 15) != 0 || (reinterpret_cast<uintptr_t>(summaries) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(q) & 1) != 0 || (reinterpret_cast<uintptr_t>(chunks) & 3) != 0)
    return BSATTN_E_ARG;
  bsattn::ChunkParams cp{};
  cp.q = q; cp.k = k; cp.summ = summaries; cp.chunks = chunks;
  cp.q_sb = pr->q_stride[0]; cp.q_sn = pr->q_stride[1]; cp.q_sh = pr->q_stride[2];
  cp.k_sb = pr->k_stride[0]; cp.k_sn = pr->k_stride[1]; cp.k_sh = pr->k_stride[2];
  cp.B = pr->B; cp.Hq = pr->Hq; cp.Hkv = pr->Hkv; cp.Nq = pr->Nq; cp.Nk = pr->Nk; cp.d = pr->d;
  cp.grp = pr->Hq / pr->Hkv;
  cp.chunk = pr->chunk; cp.topk = pr->topk; cp.n_chunks = int32_t(n); cp.query_index = pr->query_index;
  int32_t np2 = 1;
  while (np2 < n) np2 <<= 1;
  cp.n_pad = np2;
  hipError_t e = bsattn::launch_chunk_select(cp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return BSATTN_OK;
}

int bsattn_mfma_probe(int32_t n_workgroups, int32_t iters, int32_t random, uint64_t* clocks, void* stream) {
  if (clocks == nullptr || iters < 1 || n_workgroups < 1 || n_workgroups > 65535) return BSATTN_E_ARG;
  if ((reinterpret_cast<uintptr_t>(clocks) & 7) != 0) return BSATTN_E_ARG;
  hipError_t e = bsattn::launch_mfma_probe(n_workgroups, iters, random != 0, clocks, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return BSATTN_OK;
}

int bsattn_bwd_workspace_bytes(const bsattn_plan* plan, size_t* bytes) {
  if (plan == nullptr || bytes == nullptr) return BSATTN_E_ARG;
  *bytes = bwd_workspace_bytes(plan->prob);
  return BSATTN_OK;
}

int bsattn_bwd(const bsattn_plan* plan, const void* q, const void* k, const void* v, const void* o,
               const float* lse, const void* dout, void* dq, void* dk, void* dv, float scale, void* workspace,
               size_t workspace_bytes, void* stream) {
  return run_bwd(plan, q, k, v, o, lse, dout, dq, dk, dv, scale, workspace, workspace_bytes, stream);
}

int bsattn_fwd(const bsattn_plan* plan, const void* q, const void* k, const void* v, void* o, float* lse,
               float scale, void* stream) {
  return run_fwd(plan, 0, bsattn::kShapes, q, k, v, o, lse, scale, stream);
}

int bsattn_fwd_shape(const bsattn_plan* plan, int32_t shape, const void* q, const void* k, const void* v,
                     void* o, float* lse, float scale, void* stream) {
  if (shape < 0 || shape >= bsattn::kShapes) return BSATTN_E_ARG;
  return run_fwd(plan, shape, shape + 1, q, k, v, o, lse, scale, stream);
}

int bsattn_plan_destroy(bsattn_plan* plan) {
  delete plan;
  return BSATTN_OK;
}

const char* bsattn_status_string(int status) {
  switch (status) {
    case BSATTN_OK: return "ok";
    case BSATTN_E_ARG: return "invalid argument";
    case BSATTN_E_LAYOUT: return "invalid token layout";
    case BSATTN_E_SELECTION: return "invalid block selection";
    case BSATTN_E_UNSUPPORTED: return "unsupported problem";
    case BSATTN_E_OOM: return "host out of memory";
    case BSATTN_E_HIP: return "HIP runtime error";
    case BSATTN_E_STATE: return "plan not uploaded";
    default: return "unknown status";
  }
}

int bsattn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
