// Host-side plan: K/V pages, Q-tile routing, page lists and pair counts.
//
// KPage abstract (zhuanzhiai page 1): sentence 2 -- 16-row K/V pages of valid tokens,
// packed across logical-block boundaries into large tiles while loading; sentence 3 --
// Q blocks routed between 64x256 and 128x128 tiles; sentence 4 -- pages are owned by
// one K/V block and masking is exact; sentence 7 -- physical vs useful pair capacity.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "bsattn.h"
#include "kernel_params.hpp"

namespace bsattn {

constexpr int kPage = 16;
constexpr int kShapes = 2;
constexpr int kTileRows[kShapes] = {128, 64};
constexpr int kTileCols[kShapes] = {128, 256};
constexpr int kPagesPerKTile[kShapes] = {8, 16};
// page-list entries are packed as (first slot << 5) | valid rows, plus kEntryMaskBit on the
// entries of every 4-entry stage (counted from the start of its list) that holds a partial
// page or ends past the list: stages without it need no mask for empty page rows
constexpr int kEntryShift = 5;
constexpr int64_t kMaxSlots = int64_t(1) << (31 - kEntryShift);  // slots use bits 5..30
constexpr uint32_t kEntryMaskBit = 0x80000000u;
constexpr int kStagePages = 4;
// zero entries after the page lists (kernels read up to 27 entries past a list's end)
constexpr size_t kEntryPad = 64;
constexpr size_t kPermPad = 16;
// backward tiles: 64 rows of one block on either side (two waves of 32 rows)
constexpr int kDqTileRows = 128;  // rows of a dQ tile (one Q block's slots)
constexpr int kKvTileRows = 64;   // rows of a dK/dV tile (one K block's slots)

}  // namespace bsattn

struct bsattn_plan {
  bsattn_problem prob{};
  int32_t flags = 0;  // BSATTN_PLAN_*
  std::vector<int32_t> qblock_order;  // dispatch order of Q blocks (empty: ascending)
  int32_t nqb = 0, nkb = 0, sel_nb = 1, sel_nh = 1, n_units = 1;
  // canonical arrays (exported)
  std::vector<int32_t> page_kblock, page_slot0, page_nvalid;
  std::vector<int32_t> qt_qblock, qt_row0, qt_rows, qt_shape;
  std::vector<int64_t> pl_ptr;
  std::vector<int32_t> pl_pages;
  bsattn_stats stats{};
  // device image, staged on the host; offsets are byte offsets into it
  std::vector<uint8_t> image;
  size_t off_qt[bsattn::kShapes] = {0, 0};
  int32_t n_qt[bsattn::kShapes] = {0, 0};
  int32_t n_dqt_split = 0;  // dQ tiles of at most kDqSplitRows rows (last in the device image)
  size_t off_plptr = 0, off_plent = 0, off_qperm = 0, off_kperm = 0;
  bool has_qperm = false, has_kperm = false;
  // backward: Q pages (16 valid rows of one Q block), 64-row tiles of each side, and the
  // transposed lists -- Q pages per (unit, K block), Q blocks ascending, pages ascending
  std::vector<int32_t> qpage_qblock, qpage_slot0, qpage_nvalid;
  std::vector<int32_t> dqt_qblock, dqt_row0, dqt_rows;
  std::vector<int32_t> kvt_kblock, kvt_row0, kvt_rows;
  std::vector<int64_t> tpl_ptr;
  std::vector<int32_t> tpl_pages;
  size_t off_dqt = 0, off_kvt = 0, off_tplptr = 0, off_tplent = 0;
  // device-side selection updates: the K layout's first page per block and packed page
  // words, and the capacity of the entry array
  size_t off_firstpage = 0, off_pageent = 0;
  int64_t ent_capacity = 0;
  // the same for the transposed lists: the Q layout's first page per block, packed Q page
  // words, and the capacity of the transposed entry array
  size_t off_firstqpage = 0, off_qpageent = 0;
  int64_t tent_capacity = 0;
  // bound device buffer (caller-owned)
  void* dev = nullptr;
};

namespace bsattn {
// Builds *p from validated arguments; returns a bsattn_status.
// flags: BSATTN_PLAN_* (0 = the packed plan)
int build_plan(const bsattn_problem& prob, const bsattn_layout& ql, const bsattn_layout& kl,
               const bsattn_selection& sel, int32_t flags, bsattn_plan* p);
// Writes the forward Q-tile tables of the device image in dispatch order.
void write_qtiles(bsattn_plan* p);
// Validates a permutation of the Q blocks and makes it the dispatch order.
int set_block_order(bsattn_plan* p, const int32_t* order, int32_t n);
}  // namespace bsattn
