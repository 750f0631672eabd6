// Arguments of the forward and backward kernels (passed by value) and the device tile record.
#pragma once

#include <cstddef>
#include <cstdint>

namespace bsattn {

// dQ tiles of at most this many rows (two 32-row groups) split their keys over the waves
constexpr int kDqSplitRows = 64;

// XCDs (of the chip's 8) that work on one (batch, head) slice of the forward at a time.
constexpr int kXcdShare = 1;

// One Q tile as the kernel reads it.
struct QTileDev {
  int32_t row0;    // first slot in the Q layout
  int32_t rows;    // valid rows
  int32_t qblock;  // Q block id
  int32_t pad;
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_sn, q_sh;
  int64_t k_sb, k_sn, k_sh;
  int64_t v_sb, v_sn, v_sh;
  int64_t o_sb, o_sn, o_sh;
  const QTileDev* qtiles;     // Q tiles of one shape (the 128-row tiles in a launch of both)
  const QTileDev* qtiles2;    // a launch of both shapes: the 64-row tiles
  const int32_t* pl_ptr;      // [n_units * nqb + 1]
  const int32_t* pl_ent;      // packed (first slot << 5) | valid rows
  const int32_t* qperm;       // slot -> token, or null
  const int32_t* kperm;
  int64_t q_pos0;
  uint32_t k_extent, v_extent;  // bytes of one (batch, KV head) slice reachable from its base
  uint32_t k_sn_bytes, v_sn_bytes;
  int32_t n_qtiles;           // tiles of this shape
  int32_t n_work;             // n_qtiles * B * Hq
  int32_t n_qtiles2, n_work2; // a launch of both shapes: the same for the 64-row tiles
  int32_t B, Hq, Hkv, Nq, Nk, grp;
  int32_t nqb, sel_nh, ub_mul, uh_div;
  int32_t causal;
  float scale, scale_log2;
};

// Backward.  Gradients share the layout of their tensors: dO uses O's strides, dQ Q's, dK
// K's and dV V's.  D = rowsum(dO * O) lives in a float32 [B, Hq, Nq] workspace.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // [B, Hq, Nq], natural log
  void* dq;
  void* dk;
  void* dv;
  float* dvec;       // workspace: D [B, Hq, Nq]
  int64_t q_sb, q_sn, q_sh;
  int64_t k_sb, k_sn, k_sh;
  int64_t v_sb, v_sn, v_sh;
  int64_t o_sb, o_sn, o_sh;
  const QTileDev* dq_tiles;   // 128-row Q tiles (row0, rows, qblock): the last n_dq_split
                              // hold at most kDqSplitRows rows
  const QTileDev* kv_tiles;   // 64-row K tiles (first slot, rows, kblock)
  const int32_t* pl_ptr;      // K pages per (unit, Q block), as in the forward
  const int32_t* pl_ent;
  const int32_t* tpl_ptr;     // Q pages per (unit, K block): [n_units * nkb + 1]
  const int32_t* tpl_ent;     // packed (first slot << 5) | valid rows
  const int32_t* qperm;
  const int32_t* kperm;
  int64_t q_pos0;
  uint32_t q_extent, o_extent, k_extent, v_extent;  // bytes of one (batch, head) slice
  uint32_t q_sn_bytes, o_sn_bytes, k_sn_bytes, v_sn_bytes;
  int32_t n_dq_tiles, n_kv_tiles, n_dq_split;
  int32_t B, Hq, Hkv, Nq, Nk, grp;
  int32_t nqb, nkb, sel_nh, ub_mul, uh_div;
  int32_t causal;
  float scale, scale_log2;
};

// Decode / small query blocks: the query heads of a KV group stacked into one 32-column
// tile per Q block, pages split over workgroups, partial softmax states merged after.
struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_sn, q_sh;
  int64_t k_sb, k_sn, k_sh;
  int64_t v_sb, v_sn, v_sh;
  int64_t o_sb, o_sn, o_sh;
  const QTileDev* qtiles;  // one tile per Q block (every block has at most 32 / grp rows)
  const int32_t* pl_ptr;
  const int32_t* pl_ent;
  const int32_t* qperm;
  const int32_t* kperm;
  float* opart;   // workspace: [work][32][d] unnormalised O of a split
  float* mlpart;  // workspace: [work][32][2] running max (log2 units) and sum of a split
  int64_t q_pos0;
  uint32_t k_extent, v_extent, k_sn_bytes, v_sn_bytes;
  int32_t n_qtiles, n_splits, pps;  // tiles, splits per (b, g, tile), pages per split (multiple of 8)
  int32_t B, Hq, Hkv, Nq, Nk, grp;
  int32_t nqb, sel_nh, ub_mul, uh_div;
  int32_t causal;
  float scale, scale_log2;
};

// Bytes of the library-held device buffer behind bsattn_fwd_decode_noalloc (per GPU).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;

// Page lists rebuilt on the device from a device-resident selection.
struct PlanUpdateParams {
  const int32_t* row_ptr;     // [n_rows + 1] selection CSR (device)
  const int32_t* kblk;        // selected K block ids, strictly ascending per row
  const int32_t* first_page;  // [nkb + 1] first page of each K block
  const int32_t* page_ent;    // [n_pages] packed page words
  int32_t* pl_ptr;            // [n_rows + 1] row pointers of the plan
  int32_t* pl_ent;            // [capacity] entries of the plan
  int32_t* status;            // |= 1 capacity exceeded, 2 block id out of range, 4 row not ascending
  int32_t n_rows, nkb, capacity;
  // transposed lists (backward): Q pages per (unit, K block), Q blocks ascending
  const int32_t* first_qpage; // [nqb + 1] first page of each Q block
  const int32_t* qpage_ent;   // [n_qpages] packed Q page words
  int32_t* tpl_ptr;           // [n_units * nkb + 1]
  int32_t* tpl_ent;           // [tcapacity]
  int32_t n_units, nqb, tcapacity;
};

// Chunk selection: summaries of key chunks and the top-k chunks per (batch, KV group).
struct ChunkParams {
  const void* q;
  const void* k;
  float* summ;      // [B, Hkv, n_chunks, d] float32
  int32_t* chunks;  // [B, Hkv, topk], ascending chunk ids
  int64_t q_sb, q_sn, q_sh;
  int64_t k_sb, k_sn, k_sh;
  int32_t B, Hq, Hkv, Nq, Nk, d, grp;
  int32_t chunk, topk, n_chunks, n_pad, query_index;
};

}  // namespace bsattn
