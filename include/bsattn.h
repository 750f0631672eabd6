/*
 * bsattn -- exact block-sparse softmax attention (forward and backward) for AMD MI355X (gfx950).
 *
 * The operation (KPage abstract, zhuanzhiai page 1, sentences 2-4; FlashAttention
 * entries of the scifaro related-paper lists for the softmax / log-sum-exp convention):
 *
 *   For batch b, query head h (KV head g = h / (Hq / Hkv)), query token i and key token j,
 *   the pair (i, j) is in the sparse graph iff the K block holding j is in the selected
 *   set of the Q block holding i (for the selection unit of (b, h)) and, when the problem
 *   is causal, j <= q_pos0 + i.  Then
 *       O[b, i, h, :] = sum_j softmax_j(scale * <Q[b,i,h,:], K[b,j,g,:]>) V[b, j, g, :]
 *       LSE[b, h, i]  = ln sum_j exp(scale * <Q[b,i,h,:], K[b,j,g,:]>)
 *   over the graph's keys only.  A query with no key gets O = 0 and LSE = -inf.
 *
 * How it is computed (same abstract, sentences 2-3): every K block is cut into 16-row
 * pages of valid tokens, each owned by that block; the pages selected by a Q block are
 * packed, across block boundaries, into K tiles of 8 pages (128 keys) or 16 pages
 * (256 keys) as they are loaded into LDS -- no compacted copy is written to HBM.  Q
 * blocks are routed between 128-row tiles (128x128) and 64-row tiles (64x256) so that a
 * small Q block does not pad to 128 rows.  Masking is exact: empty page slots, padded
 * query rows and causally hidden keys never contribute.
 *
 * Conventions
 *   - Every call returns an int status: BSATTN_OK (0) or one of the BSATTN_E_* codes.
 *     No C++ exception crosses this interface.  bsattn_status_string() names a code.
 *   - Host arrays passed in (layouts, selections) are read during the call only.
 *   - All device memory is owned by the caller: the library never allocates device
 *     memory.  Streams are hipStream_t values passed as void* (NULL = default stream).
 *   - A plan is immutable once uploaded and may be used from several host threads;
 *     bsattn_fwd calls that share a plan may run concurrently on different streams.
 */
#ifndef BSATTN_H_
#define BSATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bsattn_status {
  BSATTN_OK = 0,
  BSATTN_E_ARG = 1,          /* null pointer, bad size or count, plan/argument mismatch */
  BSATTN_E_LAYOUT = 2,       /* offsets not rising from 0 to N, or perm not a permutation */
  BSATTN_E_SELECTION = 3,    /* selection CSR malformed or a block id out of range */
  BSATTN_E_UNSUPPORTED = 4,  /* head_dim not 64/128, dtype not bf16, page size not 16, sizes past limits */
  BSATTN_E_OOM = 5,          /* host allocation failed */
  BSATTN_E_HIP = 6,          /* a HIP runtime call failed (see bsattn_last_hip_error) */
  BSATTN_E_STATE = 7         /* plan not uploaded to device memory */
};

enum { BSATTN_DTYPE_BF16 = 1 };

/* Tile shapes (KPage abstract, sentence 3): rows of the Q tile x columns of the K tile. */
enum { BSATTN_SHAPE_128x128 = 0, BSATTN_SHAPE_64x256 = 1 };

/* Problem shape.  Tensors are Q [B, Nq, Hq, d], K and V [B, Nk, Hkv, d], O like Q, all
 * bf16 with d contiguous; the *_stride arrays give the element strides of the batch,
 * token and head dimensions.  LSE is float32 [B, Hq, Nq], contiguous.  For a causal
 * problem, query token i sits at absolute position q_pos0 + i and key token j at j. */
typedef struct bsattn_problem {
  int32_t B, Hq, Hkv, Nq, Nk, d;
  int32_t dtype;     /* BSATTN_DTYPE_BF16 */
  int32_t causal;    /* 0 or 1 */
  int64_t q_pos0;
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
} bsattn_problem;

/* Token layout of one side, shared by every batch and head.  Block k holds the slots
 * [offsets[k], offsets[k+1]); slot s holds token perm[s] (token s when perm is NULL).
 * offsets must rise from 0 to N; perm, when given, must be a permutation of [0, N).
 * Empty blocks are allowed. */
typedef struct bsattn_layout {
  int32_t n_blocks;
  const int32_t* offsets; /* [n_blocks + 1] */
  const int32_t* perm;    /* [N] or NULL */
} bsattn_layout;

/* Block selection as CSR over rows (unit, Q block), row = unit * n_qblocks + qblock,
 * unit = ub * n_h + uh.  n_b is 1 (shared by all batches, ub = 0) or B (ub = b).  n_h is
 * Hq (uh = h), Hkv (uh = h / (Hq/Hkv): one selection per KV group, shared by the group's
 * query heads -- CISA abstract, fugumt page 4, sentence 4) or 1 (uh = 0).  When Hq equals
 * Hkv the two readings coincide.  A row lists selected K block ids in any order;
 * duplicates count once. */
typedef struct bsattn_selection {
  int32_t n_b, n_h;
  const int32_t* row_ptr; /* [n_b * n_h * n_qblocks + 1], rising from 0 */
  const int32_t* kblk;    /* [row_ptr[last]], each in [0, n_kblocks) */
} bsattn_selection;

/* Plan statistics (KPage abstract, sentence 7: useful vs physical query-key pairs).
 * useful   = pairs of the sparse graph over all (batch, head), causal exclusions removed;
 * physical = sum over (batch, head) and Q tiles of tile_rows * tile_cols * K tiles,
 *            padded rows and empty page slots included. */
typedef struct bsattn_stats {
  int64_t useful;
  int64_t physical;
  int64_t n_pages;        /* K pages of the layout */
  int64_t n_qtiles128;    /* Q tiles of the layout routed to 128x128 */
  int64_t n_qtiles64;     /* Q tiles of the layout routed to 64x256 */
  int64_t n_ktiles;       /* K tiles over all (batch, head, Q tile) work items */
  int64_t page_list_len;  /* entries of all (unit, Q block) page lists */
  int64_t n_units;        /* selection units */
  int64_t useful_by_shape[2];    /* useful pairs in tiles of each shape (BSATTN_SHAPE_*) */
  int64_t physical_by_shape[2];  /* physical pairs in tiles of each shape */
} bsattn_stats;

/* Canonical plan arrays (views into plan memory, valid until bsattn_plan_destroy).
 * Pages are ordered by K block then page; a page id indexes page_*.  Q tiles are
 * ordered by Q block then row.  pl_ptr/pl_pages give each (unit, Q block) row's page
 * ids: selected blocks ascending, each block's pages ascending. */
typedef struct bsattn_plan_view {
  int64_t n_pages;
  const int32_t* page_kblock;
  const int32_t* page_slot0;  /* first slot of the page in the K layout */
  const int32_t* page_nvalid; /* 1..16 */
  int64_t n_qtiles;
  const int32_t* qt_qblock;
  const int32_t* qt_row0;     /* first slot of the tile in the Q layout */
  const int32_t* qt_rows;     /* valid rows */
  const int32_t* qt_shape;    /* BSATTN_SHAPE_* */
  int64_t n_rows;             /* n_units * n_qblocks */
  const int64_t* pl_ptr;      /* [n_rows + 1] */
  const int32_t* pl_pages;    /* [pl_ptr[n_rows]] */
} bsattn_plan_view;

/* Backward tables of a plan (views into plan memory, valid until bsattn_plan_destroy).
 * Q pages: each Q block of n slots has ceil(n/16) pages of 16 valid rows (the last may be
 * short), ordered by Q block then page.  Owned tiles of one block on each side, ordered
 * by block then row: 128 slots per dQ tile of a Q block and 64 per dK/dV tile of a K block
 * (ceil(n/height) per block, the last one short).  tpl_ptr/tpl_pages
 * give, for each (unit, K block) row = unit * n_kblocks + kblock, the Q page ids of every Q
 * block whose selection holds that K block: Q blocks ascending, each block's pages
 * ascending (KPage abstract, sentence 4: the K/V side owns its rows in backward). */
typedef struct bsattn_plan_bwd_view {
  int64_t n_qpages;
  const int32_t* qpage_qblock;
  const int32_t* qpage_slot0;  /* first slot of the page in the Q layout */
  const int32_t* qpage_nvalid; /* 1..16 */
  int64_t n_dq_tiles;
  const int32_t* dqt_qblock;
  const int32_t* dqt_row0;     /* first slot in the Q layout */
  const int32_t* dqt_rows;     /* 1..128 */
  int64_t n_kv_tiles;
  const int32_t* kvt_kblock;
  const int32_t* kvt_row0;     /* first slot in the K layout */
  const int32_t* kvt_rows;     /* 1..64 */
  int64_t n_trows;             /* n_units * n_kblocks */
  const int64_t* tpl_ptr;      /* [n_trows + 1] */
  const int32_t* tpl_pages;    /* [tpl_ptr[n_trows]] Q page ids */
} bsattn_plan_bwd_view;

typedef struct bsattn_plan bsattn_plan;

/* Build a plan on the host: validate, cut K blocks into pages, route Q blocks into
 * tiles, build the page lists and the pair counts.  page_size must be 16.  On success
 * *out owns a new plan (free it with bsattn_plan_destroy); on failure *out is NULL.
 * Limits (BSATTN_E_UNSUPPORTED past them): Nq, Nk < 2^26; B * Hq <= 2^24; selection units times Q blocks,
 * and selection units times K blocks, below 2^31 - 1; page lists (forward and transposed)
 * below 2^31 entries. */
int bsattn_plan_create(const bsattn_problem* problem, const bsattn_layout* q_layout,
                       const bsattn_layout* k_layout, const bsattn_selection* selection,
                       int32_t page_size, bsattn_plan** out);

/* Plan flags for bsattn_plan_create_ex. */
enum {
  /* The fixed-tile baseline that page packing and Q routing are measured against (KPage
   * abstract, sentences 5 and 7: speedup over NVIDIA BSA, physical pair capacity): every
   * Q tile has 128 rows (no 64x256 routing) and every selected K block starts a new
   * 128-key tile, padded with empty page slots -- one 128x128 tile per (Q block, selected
   * K block) pair for blocks of at most 128 tokens.  Same results, more physical pairs. */
  BSATTN_PLAN_FIXED_TILES = 1
};

/* bsattn_plan_create with flags (0 gives the same plan as bsattn_plan_create); unknown
 * flag bits are BSATTN_E_ARG.  In a BSATTN_PLAN_FIXED_TILES plan the exported page lists
 * hold -1 for the empty padding slots. */
int bsattn_plan_create_ex(const bsattn_problem* problem, const bsattn_layout* q_layout,
                          const bsattn_layout* k_layout, const bsattn_selection* selection,
                          int32_t page_size, int32_t flags, bsattn_plan** out);

/* Dispatch order of the forward's Q tiles: order[i] is the i-th Q block whose tiles are
 * launched (a permutation of [0, n_qblocks); each block's tiles stay in row order).  A
 * locality hint only -- results do not change: Q tiles that run at the same time on one XCD
 * and walk overlapping page lists at similar offsets share that XCD's L2.  The default is
 * ascending block order.  It takes effect at the next bsattn_plan_upload.  Errors:
 * BSATTN_E_ARG if order is not such a permutation. */
int bsattn_plan_set_block_order(bsattn_plan* plan, const int32_t* order, int32_t n_qblocks);

/* Bytes of device memory the plan needs (a multiple of 256). */
int bsattn_plan_device_bytes(const bsattn_plan* plan, size_t* bytes);

/* Copy the plan's device tables into dev (caller-owned device memory of at least
 * bsattn_plan_device_bytes bytes, 256-byte aligned) on stream, asynchronously.  The
 * host copy stays valid; dev must stay alive while the plan is used.  Uploading again
 * rebinds the plan to the new buffer. */
int bsattn_plan_upload(bsattn_plan* plan, void* dev, size_t bytes, void* stream);

/* Rebuild the plan's page lists on the device from a device-resident selection (a mask
 * that changes every step, such as the chunks of bsattn_chunk_select), asynchronously on
 * stream, with the host planner's rules (selected blocks ascending, pages ascending, stage
 * flags), then the backward's transposed lists (for each unit and K block, the Q pages of
 * the Q blocks that select it, Q blocks ascending).  n_b and n_h must match the plan's
 * selection; row_ptr [n_b * n_h * n_qblocks + 1] and kblk are device int32 arrays, each row
 * strictly ascending (bsattn_chunk_select's output is).  Each set of lists may hold at most
 * as many entries as it held for the selection the plan was created with (page_list_len for
 * the forward lists); longer lists are cut at that capacity.  status, if not NULL, is a
 * device int32 that the update ORs with 1 (a capacity exceeded), 2 (a block id out of range,
 * skipped) or 4 (a row not strictly ascending); the caller clears it.  Afterwards bsattn_fwd,
 * bsattn_fwd_shape, bsattn_fwd_decode and bsattn_bwd use the new lists (calls ordered on
 * the stream); the host-side statistics and exported arrays keep the creation selection.
 * bsattn_plan_upload restores the creation selection.  BSATTN_E_UNSUPPORTED for a plan made
 * with flags. */
int bsattn_plan_update_selection(bsattn_plan* plan, int32_t n_b, int32_t n_h, const int32_t* row_ptr,
                                 const int32_t* kblk, int32_t* status, void* stream);

int bsattn_plan_stats(const bsattn_plan* plan, bsattn_stats* stats);

int bsattn_plan_export(const bsattn_plan* plan, bsattn_plan_view* view);

/* The backward tables (see bsattn_plan_bwd_view), for the bit-exact planner tests. */
int bsattn_plan_export_bwd(const bsattn_plan* plan, bsattn_plan_bwd_view* view);

/* The forward pass: O and LSE for every (batch, query, head), asynchronously on stream.
 * q, k, v, o: device bf16 tensors laid out as the problem's strides say (16-byte aligned
 * rows); lse: device float32 [B, Hq, Nq]; scale: the softmax scale, finite and > 0.  Every
 * O row and LSE entry is written.  No allocation, no synchronisation.  Strides must be
 * non-negative, and the K (and V) rows of one (batch, KV head) must lie within 4 GiB of
 * that slice's first element (BSATTN_E_UNSUPPORTED otherwise).  K and V must be finite in
 * every row of the key layout, selected or not: page rows past a block's end and empty page
 * slots load some row of the slice and get probability exactly 0, and 0 times an infinite
 * V entry would be NaN.  Returns BSATTN_E_STATE when the plan was never uploaded,
 * BSATTN_E_ARG on a null or misaligned pointer, BSATTN_E_HIP on a launch error. */
int bsattn_fwd(const bsattn_plan* plan, const void* q, const void* k, const void* v, void* o,
               float* lse, float scale, void* stream);

/* The part of bsattn_fwd that covers the Q tiles of one shape (BSATTN_SHAPE_128x128 or
 * BSATTN_SHAPE_64x256, KPage abstract sentence 3): one kernel launch on stream.  The two
 * shapes write disjoint rows of O and LSE, so calling both -- in either order, on one
 * stream or on two -- is the same as one bsattn_fwd call.  Same arguments, ownership
 * and errors as bsattn_fwd; an unknown shape is BSATTN_E_ARG. */
int bsattn_fwd_shape(const bsattn_plan* plan, int32_t shape, const void* q, const void* k, const void* v,
                     void* o, float* lse, float scale, void* stream);

/* Backward workspace: bytes of device memory bsattn_bwd needs for D = rowsum(dO * O),
 * float32 [B, Hq, Nq] (a multiple of 256, at least 256). */
int bsattn_bwd_workspace_bytes(const bsattn_plan* plan, size_t* bytes);

/* The backward pass: gradients of the same masked softmax attention (KPage abstract,
 * sentence 4: the backward works on the selected pairs only, with pages owned by one K/V
 * block).  With P^ = exp(scale <Q_i, K_j> - LSE_i) on the graph's pairs and 0 elsewhere,
 * dO the gradient of O and D_i = sum_e dO_ie O_ie:
 *     dV[b, j, g, :] = sum over the query heads h of group g, sum_i P^_ij dO[b, i, h, :]
 *     dS_ij          = P^_ij (<dO[b, i, h, :], V[b, j, g, :]> - D_i)
 *     dQ[b, i, h, :] = scale sum_j dS_ij K[b, j, g, :]
 *     dK[b, j, g, :] = scale sum over h of group g, sum_i dS_ij Q[b, i, h, :]
 * Inputs: q, k, v as for bsattn_fwd; o and lse as bsattn_fwd wrote them for the same
 * inputs; dout: bf16 dO laid out with O's strides.  Outputs (bf16, fully overwritten): dq
 * with Q's strides, dk with K's, dv with V's; keys that no query reaches and queries with no
 * key get zeros.  workspace: caller-owned device memory of at least
 * bsattn_bwd_workspace_bytes bytes (16-byte aligned), overwritten.  Each dK/dV row is
 * produced by the one workgroup that owns its key, each dQ row by the one that owns its
 * query: no atomics, and the result is the same on every call.  Asynchronous on stream; no
 * allocation, no synchronisation.  The Q and dO rows of one (batch, query head) must lie
 * within 4 GiB of the slice's first element, like K and V, and the plan's transposed page
 * lists (bsattn_plan_export_bwd) must hold fewer than 2^29 - 64 entries
 * (BSATTN_E_UNSUPPORTED otherwise).  Q, K, V and dO must be finite in every row of their layouts.  Errors as for
 * bsattn_fwd; a missing or short workspace is BSATTN_E_ARG. */
int bsattn_bwd(const bsattn_plan* plan, const void* q, const void* k, const void* v, const void* o,
               const float* lse, const void* dout, void* dq, void* dk, void* dv, float scale,
               void* workspace, size_t workspace_bytes, void* stream);

/* Decode and other small query blocks (the same operation as bsattn_fwd).  When every Q
 * block has at most 32 / (Hq / Hkv) rows and the query heads of a KV group share their
 * selection unit (selection n_h = 1 or Hkv), the group's heads are stacked into the 32
 * columns of one tile per Q block, so each selected K/V page is read once per group instead
 * of once per head (CISA abstract, fugumt page 4, sentences 4-5: one indexing query per KV
 * group, selections shared by the group's queries).  Each page list is split over many
 * workgroups and the partial softmax states are merged exactly.  Same arguments as
 * bsattn_fwd plus a caller-owned device workspace of at least bsattn_decode_workspace_bytes
 * bytes (16-byte aligned; it holds the partial states).  Two launches, no allocation.
 * BSATTN_E_UNSUPPORTED when the plan does not meet the conditions above (or was made with
 * flags); other errors as for bsattn_fwd. */
int bsattn_decode_workspace_bytes(const bsattn_plan* plan, size_t* bytes);
int bsattn_fwd_decode(const bsattn_plan* plan, const void* q, const void* k, const void* v, void* o,
                      float* lse, float scale, void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving
 * loops, harnesses that forbid hipMalloc): bsattn_fwd_decode with the partial states in a
 * buffer the library holds in its own device data, 16 MiB per GPU (kept until the process
 * ends), instead of a caller workspace.  Allocates nothing.  Every call on one GPU uses that
 * GPU's one buffer: calls that overlap on a GPU (on different streams, or from different
 * threads) race and must be ordered by the caller; each call writes every partial state it
 * reads, so nothing carries over from an earlier call.  Same arguments (without the
 * workspace), results and errors as bsattn_fwd_decode; BSATTN_E_UNSUPPORTED also when
 * bsattn_decode_workspace_bytes exceeds 16 MiB (checked before the upload state). */
int bsattn_fwd_decode_noalloc(const bsattn_plan* plan, const void* q, const void* k, const void* v, void* o,
                              float* lse, float scale, void* stream);

/* Chunk selection (CISA abstract, fugumt page 4, sentences 3-5: fixed-size KV chunks
 * chosen with compact summaries of the keys, one indexing query per KV group, the selection
 * shared by the group's queries).  Q [B, Nq, Hq, d] and K [B, Nk, Hkv, d] are bf16 with the
 * given element strides (d contiguous, K rows 16-byte aligned).  Chunk c holds key tokens
 * [c * chunk, min(Nk, (c + 1) * chunk)); n_chunks = ceil(Nk / chunk).  For each batch b and
 * KV group g:
 *     summary[b, g, c] = mean of the chunk's keys (float32)
 *     iq[b, g]         = mean over the group's query heads of Q[b, query_index, h, :]
 *     score            = <summary, iq>
 * and the topk highest-scoring chunks (ties to the lower chunk id) are written to
 * chunks[b, g, :] in ascending order.  In an attention problem they form the selection
 * row of unit (b, g) (selection n_b = B, n_h = Hkv) for a Q block of the queries that share
 * it.  summaries: caller-owned device float32 [B, Hkv, n_chunks, d], written (16-byte
 * aligned); chunks: caller-owned device int32 [B, Hkv, topk], written.  Asynchronous on
 * stream, two kernel launches, no allocation.  Errors: BSATTN_E_ARG for null or misaligned
 * pointers, Hq not a multiple of Hkv, query_index outside [0, Nq) or topk outside
 * [1, n_chunks]; BSATTN_E_UNSUPPORTED for d not 64/128 or n_chunks > 8192; BSATTN_E_HIP on
 * a launch error. */
typedef struct bsattn_chunk_problem {
  int32_t B, Hq, Hkv, Nq, Nk, d;
  int32_t chunk;        /* key tokens per chunk */
  int32_t topk;         /* chunks kept per (batch, KV group) */
  int32_t query_index;  /* the query row whose heads form the indexing query */
  int32_t reserved;     /* 0 */
  int64_t q_stride[3];
  int64_t k_stride[3];
} bsattn_chunk_problem;

int bsattn_chunk_select(const bsattn_chunk_problem* problem, const void* q, const void* k, float* summaries,
                        int32_t* chunks, void* stream);

/* Dense-MFMA calibration, a measurement aid beside the attention calls: the rate at which
 * the matrix cores run the forward's product (v_mfma_f32_32x32x16_bf16, bf16 in, fp32
 * accumulate) with nothing else on the chip, for quoting a kernel's rate against what the
 * chip sustains under its power limit as well as against the nominal peak.  One kernel of
 * n_workgroups workgroups of 4 waves (2 per CU fills every SIMD with two waves); each wave
 * issues iters x 32 products on register operands (1,048,576 FLOPs per wave and iteration),
 * pseudo-random bf16 of unit-normal-like spread when random != 0, zeros otherwise.  The
 * first wave of workgroup i writes clocks[2 i] = shader-clock cycles and clocks[2 i + 1] =
 * 100 MHz real-time ticks spent in its loop; the caller times the launch (FLOPs =
 * n_workgroups x 4 x iters x 32 x 32768) and takes the mean shader clock as the sum of the
 * cycle spans over the sum of the tick spans x 100 MHz.  clocks: caller-owned device
 * memory of 16 x n_workgroups bytes, 8-byte aligned, written.  Asynchronous on stream; no
 * allocation.  Errors: BSATTN_E_ARG (null or misaligned clocks, iters < 1, n_workgroups
 * outside 1..65535), BSATTN_E_HIP on a launch error. */
int bsattn_mfma_probe(int32_t n_workgroups, int32_t iters, int32_t random, uint64_t* clocks, void* stream);

int bsattn_plan_destroy(bsattn_plan* plan);

const char* bsattn_status_string(int status);

/* The hipError_t of the most recent BSATTN_E_HIP on this thread (0 if none). */
int bsattn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H_ */
