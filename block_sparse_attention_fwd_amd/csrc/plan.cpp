// Host planner.  Rules (a reading of KPage abstract sentences 2-4 and 7, zhuanzhiai page 1):
//   selection  a (unit, Q block) row selects a set of K blocks (sorted, duplicates dropped);
//   pages      a K block of n slots has ceil(n/16) pages, page p covering its slots
//              [16p, min(16p+16, n)); empty blocks have none;
//   routing    a Q block of n rows gives floor(n/128) 128-row tiles, then one 64-row tile
//              when 0 < n mod 128 <= 64, or one more 128-row tile when n mod 128 > 64;
//   K tiles    a Q tile's page list (selected blocks ascending, pages ascending) is cut
//              into ceil(pages / pages-per-tile) tiles of 8 (128x128) or 16 (64x256) pages;
//   counts     useful = graph pairs; physical = tile rows x tile cols x K tiles, summed
//              over every (batch, head) and Q tile.
// With BSATTN_PLAN_FIXED_TILES (the fixed-tile baseline the abstract compares against,
// sentences 5 and 7): every Q tile has 128 rows (ceil(n/128) per block, no 64-row tiles),
// and each selected K block starts a new K tile: its pages are followed by empty slots up
// to a multiple of 8 entries, so no tile packs pages of two blocks.
#include "plan.hpp"

#include <algorithm>
#include <cstring>
#include <new>

namespace bsattn {
namespace {

int check_layout(const bsattn_layout& l, int32_t n_tokens, std::vector<int32_t>* token_of_slot) {
  if (l.n_blocks < 0 || l.offsets == nullptr) return BSATTN_E_ARG;
  if (l.offsets[0] != 0 || l.offsets[l.n_blocks] != n_tokens) return BSATTN_E_LAYOUT;
  for (int32_t b = 0; b < l.n_blocks; ++b)
    if (l.offsets[b + 1] < l.offsets[b]) return BSATTN_E_LAYOUT;
  token_of_slot->resize(size_t(n_tokens));
  if (l.perm == nullptr) {
    for (int32_t s = 0; s < n_tokens; ++s) (*token_of_slot)[s] = s;
    return BSATTN_OK;
  }
  std::vector<uint8_t> seen(size_t(n_tokens), 0);
  for (int32_t s = 0; s < n_tokens; ++s) {
    int32_t t = l.perm[s];
    if (t < 0 || t >= n_tokens || seen[t]) return BSATTN_E_LAYOUT;
    seen[t] = 1;
    (*token_of_slot)[s] = t;
  }
  return BSATTN_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

void write_qtiles(bsattn_plan* p) {
  // dispatch order: Q blocks in p->qblock_order (ascending when empty), each block's tiles in
  // row order; the canonical (exported) tile arrays keep Q-block order
  std::vector<int32_t> rank(size_t(p->nqb));
  for (int32_t i = 0; i < p->nqb; ++i) rank[size_t(i)] = i;
  if (!p->qblock_order.empty())
    for (int32_t i = 0; i < p->nqb; ++i) rank[size_t(p->qblock_order[size_t(i)])] = i;
  for (int sh = 0; sh < kShapes; ++sh) {
    std::vector<size_t> ord;
    for (size_t t = 0; t < p->qt_shape.size(); ++t)
      if (p->qt_shape[t] == sh) ord.push_back(t);
    std::stable_sort(ord.begin(), ord.end(),
                     [&](size_t a, size_t b) { return rank[size_t(p->qt_qblock[a])] < rank[size_t(p->qt_qblock[b])]; });
    QTileDev* q = reinterpret_cast<QTileDev*>(p->image.data() + p->off_qt[sh]);
    int32_t i = 0;
    for (size_t t : ord) q[i++] = QTileDev{p->qt_row0[t], p->qt_rows[t], p->qt_qblock[t], 0};
  }
}

int set_block_order(bsattn_plan* p, const int32_t* order, int32_t n) {
  if (n != p->nqb || (n > 0 && order == nullptr)) return BSATTN_E_ARG;
  std::vector<uint8_t> seen(size_t(n), 0);
  for (int32_t i = 0; i < n; ++i) {
    if (order[i] < 0 || order[i] >= n || seen[size_t(order[i])]) return BSATTN_E_ARG;
    seen[size_t(order[i])] = 1;
  }
  p->qblock_order.assign(order, order + n);
  write_qtiles(p);
  return BSATTN_OK;
}

int build_plan(const bsattn_problem& prob, const bsattn_layout& ql, const bsattn_layout& kl,
               const bsattn_selection& sel, int32_t flags, bsattn_plan* p) {
  if ((flags & ~int32_t(BSATTN_PLAN_FIXED_TILES)) != 0) return BSATTN_E_ARG;
  const bool fixed = (flags & BSATTN_PLAN_FIXED_TILES) != 0;
  const int32_t B = prob.B, Hq = prob.Hq, Hkv = prob.Hkv, Nq = prob.Nq, Nk = prob.Nk;
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 0 || Nk < 0 || Hq % Hkv != 0) return BSATTN_E_ARG;
  if (prob.causal != 0 && prob.causal != 1) return BSATTN_E_ARG;
  if (prob.d != 64 && prob.d != 128) return BSATTN_E_UNSUPPORTED;
  if (prob.dtype != BSATTN_DTYPE_BF16) return BSATTN_E_UNSUPPORTED;
  if (int64_t(Nk) >= kMaxSlots || int64_t(Nq) >= kMaxSlots) return BSATTN_E_UNSUPPORTED;
  if (int64_t(B) * Hq > (int64_t(1) << 24)) return BSATTN_E_UNSUPPORTED;

  std::vector<int32_t> qtok, ktok;
  int st = check_layout(ql, Nq, &qtok);
  if (st != BSATTN_OK) return st;
  st = check_layout(kl, Nk, &ktok);
  if (st != BSATTN_OK) return st;

  const int32_t nqb = ql.n_blocks, nkb = kl.n_blocks;
  if (sel.n_b != 1 && sel.n_b != B) return BSATTN_E_SELECTION;
  if (sel.n_h != 1 && sel.n_h != Hkv && sel.n_h != Hq) return BSATTN_E_SELECTION;
  if (sel.row_ptr == nullptr) return BSATTN_E_ARG;
  const int64_t n_units = int64_t(sel.n_b) * sel.n_h;
  const int64_t n_rows = n_units * nqb;
  // kernels index the (unit, block) row pointers of either side with 32-bit arithmetic
  if (n_rows >= (int64_t(1) << 31) - 1 || n_units * nkb >= (int64_t(1) << 31) - 1) return BSATTN_E_UNSUPPORTED;
  if (sel.row_ptr[0] != 0) return BSATTN_E_SELECTION;
  for (int64_t r = 0; r < n_rows; ++r)
    if (sel.row_ptr[r + 1] < sel.row_ptr[r]) return BSATTN_E_SELECTION;
  if (sel.row_ptr[n_rows] > 0 && sel.kblk == nullptr) return BSATTN_E_ARG;
  for (int64_t e = 0; e < sel.row_ptr[n_rows]; ++e)
    if (sel.kblk[e] < 0 || sel.kblk[e] >= nkb) return BSATTN_E_SELECTION;

  p->prob = prob;
  p->flags = flags;
  p->nqb = nqb;
  p->nkb = nkb;
  p->sel_nb = sel.n_b;
  p->sel_nh = sel.n_h;
  p->n_units = int32_t(n_units);

  // pages
  std::vector<int32_t> first_page(size_t(nkb) + 1, 0);
  for (int32_t kb = 0; kb < nkb; ++kb) {
    const int32_t s0 = kl.offsets[kb], n = kl.offsets[kb + 1] - s0;
    for (int32_t pg = 0; pg * kPage < n; ++pg) {
      p->page_kblock.push_back(kb);
      p->page_slot0.push_back(s0 + pg * kPage);
      p->page_nvalid.push_back(std::min(kPage, n - pg * kPage));
    }
    first_page[kb + 1] = int32_t(p->page_kblock.size());
  }

  // Q routing
  for (int32_t qb = 0; qb < nqb; ++qb) {
    const int32_t s0 = ql.offsets[qb], n = ql.offsets[qb + 1] - s0;
    const int32_t full = n / 128, r = n % 128;
    for (int32_t t = 0; t < full; ++t) {
      p->qt_qblock.push_back(qb); p->qt_row0.push_back(s0 + 128 * t);
      p->qt_rows.push_back(128); p->qt_shape.push_back(BSATTN_SHAPE_128x128);
    }
    if (r > 0) {
      p->qt_qblock.push_back(qb); p->qt_row0.push_back(s0 + 128 * full);
      p->qt_rows.push_back(r);
      p->qt_shape.push_back(r <= 64 && !fixed ? BSATTN_SHAPE_64x256 : BSATTN_SHAPE_128x128);
    }
  }

  // page lists per (unit, Q block), and per-row selected-key totals for the counts
  p->pl_ptr.assign(size_t(n_rows) + 1, 0);
  std::vector<int32_t> row_sel;
  std::vector<std::vector<int32_t>> row_blocks(static_cast<size_t>(n_rows));
  for (int64_t r = 0; r < n_rows; ++r) {
    row_sel.assign(sel.kblk + sel.row_ptr[r], sel.kblk + sel.row_ptr[r + 1]);
    std::sort(row_sel.begin(), row_sel.end());
    row_sel.erase(std::unique(row_sel.begin(), row_sel.end()), row_sel.end());
    for (int32_t kb : row_sel) {
      for (int32_t pg = first_page[kb]; pg < first_page[kb + 1]; ++pg) p->pl_pages.push_back(pg);
      if (fixed)  // pad the block to whole 8-page tiles with empty slots (page id -1)
        for (int32_t n = first_page[kb + 1] - first_page[kb]; n % kPagesPerKTile[0] != 0; ++n) p->pl_pages.push_back(-1);
    }
    p->pl_ptr[r + 1] = int64_t(p->pl_pages.size());
    row_blocks[r] = row_sel;
  }
  if (p->pl_pages.size() >= (size_t(1) << 31)) return BSATTN_E_UNSUPPORTED;

  // useful pairs per (unit, shape): a non-causal tile holds rows * (selected keys) pairs;
  // a causal tile counts, per query, the selected keys at positions <= q_pos0 + token.
  std::vector<std::vector<int32_t>> ksorted;
  if (prob.causal) {
    ksorted.resize(size_t(nkb));
    for (int32_t kb = 0; kb < nkb; ++kb) {
      ksorted[kb].assign(ktok.begin() + kl.offsets[kb], ktok.begin() + kl.offsets[kb + 1]);
      std::sort(ksorted[kb].begin(), ksorted[kb].end());
    }
  }
  std::vector<int64_t> nk_row(size_t(n_rows), 0);
  for (int64_t r = 0; r < n_rows; ++r)
    for (int32_t kb : row_blocks[size_t(r)]) nk_row[size_t(r)] += kl.offsets[kb + 1] - kl.offsets[kb];
  const size_t nt = p->qt_qblock.size();
  std::vector<int64_t> unit_use(size_t(n_units) * kShapes, 0), unit_phys(size_t(n_units) * kShapes, 0);
  std::vector<int64_t> unit_kt(size_t(n_units), 0);
  std::vector<int64_t> qpos;
  for (int64_t u = 0; u < n_units; ++u) {
    for (size_t t = 0; t < nt; ++t) {
      const int sh = p->qt_shape[t];
      const int64_t row = u * nqb + p->qt_qblock[t];
      const int64_t npg = p->pl_ptr[size_t(row) + 1] - p->pl_ptr[size_t(row)];
      const int64_t k = (npg + kPagesPerKTile[sh] - 1) / kPagesPerKTile[sh];
      unit_kt[size_t(u)] += k;
      unit_phys[size_t(u) * kShapes + sh] += int64_t(kTileRows[sh]) * kTileCols[sh] * k;
      const auto& blocks = row_blocks[size_t(row)];
      if (blocks.empty()) continue;
      if (!prob.causal) {
        unit_use[size_t(u) * kShapes + sh] += int64_t(p->qt_rows[t]) * nk_row[size_t(row)];
        continue;
      }
      qpos.clear();
      for (int32_t s = p->qt_row0[t]; s < p->qt_row0[t] + p->qt_rows[t]; ++s) qpos.push_back(prob.q_pos0 + qtok[s]);
      std::sort(qpos.begin(), qpos.end());
      int64_t tot = 0;
      for (int32_t kb : blocks) {
        const auto& ks = ksorted[kb];
        if (ks.empty()) continue;
        if (int64_t(ks.back()) <= qpos.front()) { tot += int64_t(ks.size()) * int64_t(qpos.size()); continue; }
        if (int64_t(ks.front()) > qpos.back()) continue;
        for (int64_t qp : qpos)
          tot += int64_t(std::upper_bound(ks.begin(), ks.end(), qp,
                                          [](int64_t a, int32_t b) { return a < int64_t(b); }) - ks.begin());
      }
      unit_use[size_t(u) * kShapes + sh] += tot;
    }
  }

  // sum over every (b, h) through its unit
  const int32_t grp = Hq / Hkv;
  int64_t useful = 0, physical = 0, nkt = 0;
  int64_t use_sh[kShapes] = {0, 0}, phys_sh[kShapes] = {0, 0};
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t h = 0; h < Hq; ++h) {
      const int32_t ub = (sel.n_b == B) ? b : 0;
      const int32_t uh = (sel.n_h == Hq) ? h : (sel.n_h == Hkv ? h / grp : 0);
      const size_t u = size_t(int64_t(ub) * sel.n_h + uh);
      for (int sh = 0; sh < kShapes; ++sh) {
        use_sh[sh] += unit_use[u * kShapes + sh];
        phys_sh[sh] += unit_phys[u * kShapes + sh];
      }
      nkt += unit_kt[u];
    }
  }
  for (int sh = 0; sh < kShapes; ++sh) {
    useful += use_sh[sh];
    physical += phys_sh[sh];
    p->stats.useful_by_shape[sh] = use_sh[sh];
    p->stats.physical_by_shape[sh] = phys_sh[sh];
  }
  p->stats.useful = useful;
  p->stats.physical = physical;
  p->stats.n_pages = int64_t(p->page_kblock.size());
  p->stats.n_qtiles128 = std::count(p->qt_shape.begin(), p->qt_shape.end(), int32_t(BSATTN_SHAPE_128x128));
  p->stats.n_qtiles64 = std::count(p->qt_shape.begin(), p->qt_shape.end(), int32_t(BSATTN_SHAPE_64x256));
  p->stats.n_ktiles = nkt;
  p->stats.page_list_len = int64_t(p->pl_pages.size());
  p->stats.n_units = n_units;

  // backward tables.  Q pages: a Q block of n slots has ceil(n/16) pages, like the K side.
  // Owned tiles of each side: 128-row dQ tiles of each Q block, 64-row dK/dV tiles of each K
  // block (a block of n slots gives ceil(n/rows) tiles, the last one short).
  // Transposed lists: for each (unit, K block), the Q pages of every Q block that selects
  // it -- Q blocks ascending, pages ascending -- so the K/V tile that owns a key walks
  // exactly the queries in the graph with it (KPage abstract, sentence 4: K/V-owned pages in
  // backward execution).
  std::vector<int32_t> first_qpage(size_t(nqb) + 1, 0);
  for (int32_t qb = 0; qb < nqb; ++qb) {
    const int32_t s0 = ql.offsets[qb], n = ql.offsets[qb + 1] - s0;
    for (int32_t pg = 0; pg * kPage < n; ++pg) {
      p->qpage_qblock.push_back(qb);
      p->qpage_slot0.push_back(s0 + pg * kPage);
      p->qpage_nvalid.push_back(std::min(kPage, n - pg * kPage));
    }
    first_qpage[qb + 1] = int32_t(p->qpage_qblock.size());
    for (int32_t r = 0; r < n; r += kDqTileRows) {
      p->dqt_qblock.push_back(qb); p->dqt_row0.push_back(s0 + r); p->dqt_rows.push_back(std::min(kDqTileRows, n - r));
    }
  }
  for (int32_t kb = 0; kb < nkb; ++kb) {
    const int32_t s0 = kl.offsets[kb], n = kl.offsets[kb + 1] - s0;
    for (int32_t r = 0; r < n; r += kKvTileRows) {
      p->kvt_kblock.push_back(kb); p->kvt_row0.push_back(s0 + r); p->kvt_rows.push_back(std::min(kKvTileRows, n - r));
    }
  }
  {
    std::vector<std::vector<int32_t>> kq(size_t(n_units) * size_t(nkb));
    for (int64_t u = 0; u < n_units; ++u)
      for (int32_t qb = 0; qb < nqb; ++qb)
        for (int32_t kb : row_blocks[size_t(u * nqb + qb)]) kq[size_t(u) * nkb + kb].push_back(qb);
    p->tpl_ptr.assign(kq.size() + 1, 0);
    for (size_t r = 0; r < kq.size(); ++r) {
      for (int32_t qb : kq[r])
        for (int32_t pg = first_qpage[qb]; pg < first_qpage[qb + 1]; ++pg) p->tpl_pages.push_back(pg);
      p->tpl_ptr[r + 1] = int64_t(p->tpl_pages.size());
    }
  }
  if (p->tpl_pages.size() >= (size_t(1) << 31)) return BSATTN_E_UNSUPPORTED;

  // device image: Q tiles per shape, page-list pointers, packed page entries, perms
  size_t off = 0;
  for (int sh = 0; sh < kShapes; ++sh) {
    p->off_qt[sh] = off;
    p->n_qt[sh] = int32_t(std::count(p->qt_shape.begin(), p->qt_shape.end(), sh));
    off = align256(off + sizeof(QTileDev) * size_t(p->n_qt[sh]));
  }
  p->off_plptr = off;
  off = align256(off + sizeof(int32_t) * (size_t(n_rows) + 1));
  p->off_plent = off;
  // zero padding past the last entry: the kernel reads whole K tiles of entries at once
  off = align256(off + sizeof(int32_t) * (p->pl_pages.size() + kEntryPad));
  p->has_qperm = ql.perm != nullptr;
  p->has_kperm = kl.perm != nullptr;
  p->off_qperm = off;
  if (p->has_qperm) off = align256(off + sizeof(int32_t) * size_t(Nq));
  p->off_kperm = off;
  // zero padding past the key permutation: a kernel reads a page's 16 slots at once
  if (p->has_kperm) off = align256(off + sizeof(int32_t) * (size_t(Nk) + kPermPad));
  // backward: tiles of each side, transposed list pointers and entries (zero-padded: a
  // kernel reads a whole stage of entries at once)
  p->off_dqt = off;
  off = align256(off + sizeof(QTileDev) * p->dqt_row0.size());
  p->off_kvt = off;
  off = align256(off + sizeof(QTileDev) * p->kvt_row0.size());
  p->off_tplptr = off;
  off = align256(off + sizeof(int32_t) * p->tpl_ptr.size());
  p->off_tplent = off;
  off = align256(off + sizeof(int32_t) * (p->tpl_pages.size() + kEntryPad));
  // K layout tables for selection updates on the device
  p->off_firstpage = off;
  off = align256(off + sizeof(int32_t) * (size_t(nkb) + 1));
  p->off_pageent = off;
  off = align256(off + sizeof(int32_t) * p->page_kblock.size());
  p->off_firstqpage = off;
  off = align256(off + sizeof(int32_t) * (size_t(nqb) + 1));
  p->off_qpageent = off;
  off = align256(off + sizeof(int32_t) * p->qpage_qblock.size());
  p->tent_capacity = int64_t(p->tpl_pages.size());
  p->ent_capacity = int64_t(p->pl_pages.size());
  p->image.assign(std::max<size_t>(off, 256), 0);

  uint8_t* img = p->image.data();
  write_qtiles(p);
  int32_t* plp = reinterpret_cast<int32_t*>(img + p->off_plptr);
  for (size_t r = 0; r <= size_t(n_rows); ++r) plp[r] = int32_t(p->pl_ptr[r]);
  int32_t* ent = reinterpret_cast<int32_t*>(img + p->off_plent);
  for (size_t e = 0; e < p->pl_pages.size(); ++e) {
    const int32_t pg = p->pl_pages[e];
    ent[e] = pg < 0 ? 0 : (p->page_slot0[pg] << kEntryShift) | p->page_nvalid[pg];  // -1: empty slot
  }
  // mask flag: every entry of a kStagePages-entry stage (counted from its list's start) with
  // a partial page, or cut short by the list's end, carries kEntryMaskBit
  for (size_t r = 0; r < size_t(n_rows); ++r) {
    const int64_t a = p->pl_ptr[r], b = p->pl_ptr[r + 1];
    for (int64_t s0 = a; s0 < b; s0 += kStagePages) {
      const int64_t s1 = std::min<int64_t>(s0 + kStagePages, b);
      bool partial = s1 - s0 < kStagePages;
      for (int64_t e = s0; e < s1; ++e) partial |= (ent[e] & ((1 << kEntryShift) - 1)) < kPage;
      if (partial)
        for (int64_t e = s0; e < s1; ++e) ent[e] = int32_t(uint32_t(ent[e]) | kEntryMaskBit);
    }
  }
  if (p->has_qperm) std::memcpy(img + p->off_qperm, ql.perm, sizeof(int32_t) * size_t(Nq));
  if (p->has_kperm) std::memcpy(img + p->off_kperm, kl.perm, sizeof(int32_t) * size_t(Nk));
  // dQ tiles on the device: the tiles of more than kDqSplitRows rows first, then the short
  // ones (each kind in plan order), which the backward runs in a launch of their own
  QTileDev* dqt = reinterpret_cast<QTileDev*>(img + p->off_dqt);
  {
    size_t n = 0;
    for (int pass = 0; pass < 2; ++pass)
      for (size_t t = 0; t < p->dqt_row0.size(); ++t)
        if ((p->dqt_rows[t] <= kDqSplitRows) == (pass == 1))
          dqt[n++] = QTileDev{p->dqt_row0[t], p->dqt_rows[t], p->dqt_qblock[t], 0};
    p->n_dqt_split = int32_t(std::count_if(p->dqt_rows.begin(), p->dqt_rows.end(),
                                           [](int32_t r) { return r <= kDqSplitRows; }));
  }
  QTileDev* kvt = reinterpret_cast<QTileDev*>(img + p->off_kvt);
  for (size_t t = 0; t < p->kvt_row0.size(); ++t) kvt[t] = QTileDev{p->kvt_row0[t], p->kvt_rows[t], p->kvt_kblock[t], 0};
  int32_t* fpg = reinterpret_cast<int32_t*>(img + p->off_firstpage);
  for (int32_t kb = 0; kb <= nkb; ++kb) fpg[kb] = first_page[size_t(kb)];
  int32_t* pgw = reinterpret_cast<int32_t*>(img + p->off_pageent);
  for (size_t pg = 0; pg < p->page_kblock.size(); ++pg) pgw[pg] = (p->page_slot0[pg] << kEntryShift) | p->page_nvalid[pg];
  int32_t* tpp = reinterpret_cast<int32_t*>(img + p->off_tplptr);
  for (size_t r = 0; r < p->tpl_ptr.size(); ++r) tpp[r] = int32_t(p->tpl_ptr[r]);
  int32_t* tent = reinterpret_cast<int32_t*>(img + p->off_tplent);
  for (size_t e = 0; e < p->tpl_pages.size(); ++e) {
    const int32_t pg = p->tpl_pages[e];
    tent[e] = (p->qpage_slot0[pg] << kEntryShift) | p->qpage_nvalid[pg];
  }
  int32_t* fqp = reinterpret_cast<int32_t*>(img + p->off_firstqpage);
  for (int32_t qb = 0; qb <= nqb; ++qb) fqp[qb] = first_qpage[size_t(qb)];
  int32_t* qpw = reinterpret_cast<int32_t*>(img + p->off_qpageent);
  for (size_t pg = 0; pg < p->qpage_qblock.size(); ++pg) qpw[pg] = (p->qpage_slot0[pg] << kEntryShift) | p->qpage_nvalid[pg];
  return BSATTN_OK;
}

}  // namespace bsattn
