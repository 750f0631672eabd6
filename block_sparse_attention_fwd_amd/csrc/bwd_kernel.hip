// Exact block-sparse attention backward for gfx950 (MI355X).
//
// The gradients are those of masked softmax attention (KPage abstract, zhuanzhiai page 1,
// sentence 4): gradients are computed only on the pairs of the selected sparse graph, and
// every dK/dV row is owned by one K/V tile.  With P^ = exp(S - LSE) on the graph's pairs and 0 elsewhere:
//   D_i   = sum_e dO_ie O_ie                                   (bwd_dot_kernel)
//   dV_j  = sum_i P^_ij dO_i,  dK_j = scale sum_i dS_ij Q_i    (bwd_dkdv_kernel)
//   dS_ij = P^_ij (dO_i . V_j - D_i),  dQ_i = scale sum_j dS_ij K_j   (bwd_dq_kernel)
// summed over the query heads of a KV group for dK and dV.
//
// Ownership, no atomics: a dK/dV workgroup owns 64 key slots of one K block (the K/V side
// of a page never straddles blocks) and walks the transposed page list of that block -- the
// 16-row Q pages of every Q block that selects it, packed two per 32-query stage across Q
// block boundaries as they are loaded into LDS.  A dQ workgroup owns 128 query slots of one
// Q block and walks the forward's K page list of that block, two pages per 32-key stage (a
// tile of at most 64 rows gives its even and odd stages to two pairs of waves and adds the
// two partial sums at the end).
// Each wave works on 32 owned rows; the owned operands stay in registers and the streamed
// side comes through LDS.  Every product is v_mfma_f32_32x32x16_bf16 with fp32
// accumulation; P^ and dS are rounded to bf16 as MFMA operands.
//
// Per stage (32 owned x 32 streamed rows, d = 128):
//   dK/dV, score wave:    S = Q K^T, dP = dO V^T  (A = Q, dO rows from LDS; B = K^T, V^T in
//                         registers; each lane gets one key and 16 queries), P^ and dS to LDS
//   dK/dV, gradient wave: dV^T += dO^T P^, dK^T += Q^T dS  (A = dO^T, Q^T by transposing LDS
//                         reads; B = P^, dS from LDS), one stage behind the score wave
//   dQ:     S^T = K Q^T, dP^T = V dO^T (A = K, V rows; B = Q^T, dO^T in registers), then
//           dQ^T += K^T dS^T (A = K^T by transposing LDS reads)
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.hpp"
#include "kernel_params.hpp"

namespace bsattn {

template <int D>
struct BwdCfg {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;              // 16-byte chunks per row
  static constexpr int kRowsPerInst = 64 / kChunks;  // rows per 64-lane 16-byte load
  static constexpr int kInst = 16 / kRowsPerInst;    // loads per 16-row page of one tensor
  static constexpr int kStage = 32 * kRowBytes;      // 32 streamed rows of one tensor
  static constexpr int kDS = D / 16;                 // k-steps over d
  static constexpr int kDB = D / 32;                 // 32-wide d blocks of the gradients
};

constexpr float kLog2e = 1.4426950408889634f;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Consecutive work items go to one XCD (one L2): blockIdx x of n items runs item
// xcd-chunk(x & 7) + (x >> 3).
__device__ __forceinline__ int xcd_work(int blk, int n) {
  const int x = blk & 7, i = blk >> 3, q = n >> 3, r = n & 7;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// causal bound of a query position: a key token is kept iff it is <= the result
__device__ __forceinline__ int causal_thr(int64_t qpos) {
  return qpos < -1 ? -1 : (qpos > 0x7ffffffe ? 0x7ffffffe : (int)qpos);
}

// ---------------------------------------------------------------------------------------
// D = rowsum(dO * O) in fp32 from the bf16 tensors, one row per D/8 lanes.
template <int D>
__global__ void __launch_bounds__(256) bwd_dot_kernel(BwdParams p) {
  constexpr int L = D / 8;     // lanes per row
  constexpr int RPW = 64 / L;  // rows per wave
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / L;
  const int64_t nrows = (int64_t)p.B * p.Hq * p.Nq;
  float acc = 0.f;
  if (row < nrows) {
    const int64_t bh = row / p.Nq;
    const int64_t i = row - bh * p.Nq;
    const int64_t b = bh / p.Hq, h = bh - b * p.Hq;
    const int64_t off = b * p.o_sb + i * p.o_sn + h * p.o_sh + (lane % L) * 8;
    const bf16x8 o = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(p.o) + off);
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(p.dout) + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < nrows && lane % L == 0) p.dvec[row] = acc;
}

// ---------------------------------------------------------------------------------------
// Stage loads.  Wave w fills rows 16w .. 16w + 15 of a 32-row stage buffer with one 16-row
// page (first slot, valid rows) of a [tokens, d] slice.  Rows past the page's valid count
// (and a missing page) load the page's first slot: finite data that the masks remove.  Lane
// (lr, pc) of a load reads logical chunk pc ^ swz(row) of its row and stores it at physical
// chunk pc, so a wave's store of one load is a contiguous 1 KiB and the MFMA operand reads
// are conflict-free.
//
// The dK/dV kernel stages pages through registers: the loads of stage st + 2 are issued while
// stage st is computed and written to LDS in the next stage, so one barrier per stage
// separates the writes of one buffer from the reads of the others.  The dQ kernel, which keeps
// two waves per SIMD and has no registers to spare, loads pages straight into LDS one stage
// ahead.  With a permuted layout the token gather runs one stage ahead of the loads, so no
// load waits on a gather issued just before it.
template <int D>
struct PageRows {
  using C = BwdCfg<D>;
  int rip[C::kInst];
  uint32_t cb[C::kInst];
  __device__ __forceinline__ void init(int lane) {
    const int lr = lane / C::kChunks, pc = lane % C::kChunks;
#pragma unroll
    for (int n = 0; n < C::kInst; ++n) {
      rip[n] = n * C::kRowsPerInst + lr;
      cb[n] = (uint32_t)((pc ^ swz<D>(rip[n])) * 16);
    }
  }
  // tokens of the rows this lane loads for page entry ent (through perm when PERM)
  template <bool PERM>
  __device__ __forceinline__ void gather(int ent, const int32_t* perm, uint32_t (&tok)[C::kInst]) const {
    const int nv = ent_nv(ent), slot0 = ent_slot(ent);
#pragma unroll
    for (int n = 0; n < C::kInst; ++n) {
      const int slot = slot0 + (rip[n] < nv ? rip[n] : 0);
      tok[n] = (uint32_t)(PERM ? perm[slot] : slot);
    }
  }
  __device__ __forceinline__ void load(const uint32_t (&tok)[C::kInst], const __amdgpu_buffer_rsrc_t& rsrc,
                                       uint32_t sn, u32x4 (&reg)[C::kInst]) const {
#pragma unroll
    for (int n = 0; n < C::kInst; ++n)
      reg[n] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(tok[n] * sn + cb[n]), 0, 0);
  }
  // the page's rows of two tensors that share the tokens, straight into LDS
  __device__ __forceinline__ void fire(const uint32_t (&tok)[C::kInst], const __amdgpu_buffer_rsrc_t& ra,
                                       uint32_t sn_a, uint8_t* dst_a, const __amdgpu_buffer_rsrc_t& rb,
                                       uint32_t sn_b, uint8_t* dst_b, int wave) const {
#pragma unroll
    for (int n = 0; n < C::kInst; ++n) {
      const int row = 16 * wave + n * C::kRowsPerInst;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LDS_AS void*)(dst_a + row * C::kRowBytes), 16,
                                               (int)(tok[n] * sn_a + cb[n]), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (LDS_AS void*)(dst_b + row * C::kRowBytes), 16,
                                               (int)(tok[n] * sn_b + cb[n]), 0, 0, 0);
    }
  }
  // the page's rows of one tensor, straight into rows 16 page .. 16 page + 15 of dst
  __device__ __forceinline__ void fire1(const uint32_t (&tok)[C::kInst], const __amdgpu_buffer_rsrc_t& r,
                                        uint32_t sn, uint8_t* dst, int page) const {
#pragma unroll
    for (int n = 0; n < C::kInst; ++n) {
      const int row = 16 * page + n * C::kRowsPerInst;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)(dst + row * C::kRowBytes), 16,
                                               (int)(tok[n] * sn + cb[n]), 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(const u32x4 (&reg)[C::kInst], uint8_t* buf, int wave, int lane) const {
#pragma unroll
    for (int n = 0; n < C::kInst; ++n)
      *reinterpret_cast<u32x4*>(buf + (16 * wave + n * C::kRowsPerInst) * C::kRowBytes + lane * 16) = reg[n];
  }
};

// A operand of rows `row` (lane % 32) of a stage buffer, k-step s: 8 consecutive d values.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const uint8_t* buf, int lane, int s) {
  const int r = lane & 31;
  const int c = (2 * s + (lane >> 5)) ^ swz<D>(r);
  return *reinterpret_cast<const bf16x8*>(buf + r * BwdCfg<D>::kRowBytes + c * 16);
}

// A operand of the transposed stage (M = d block db, K = 16 streamed rows of half `half`)
// in the order of the accumulator layout's rows: lane l takes rows 16 half + 4 (l / 32) +
// {0..3} and the same + 8, matching a bf16x8 B operand built from accumulator registers
// 8 half .. 8 half + 7.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint8_t* buf, int lane, int half, int db) {
  using C = BwdCfg<D>;
  const int v_rr = (lane & 15) >> 2, v_qq = lane & 3, v_dsub = (lane >> 4) & 1;
  const int ra = 16 * half + 4 * (lane >> 5) + v_rr;
  const int rb = ra + 8;
  const int lc = 4 * db + 2 * v_dsub + (v_qq >> 1);
  const int off_in = (v_qq & 1) * 8;
  LDS_AS bf16x4* pa = (LDS_AS bf16x4*)(buf + ra * C::kRowBytes + ((lc ^ swz<D>(ra)) * 16) + off_in);
  LDS_AS bf16x4* pb = (LDS_AS bf16x4*)(buf + rb * C::kRowBytes + ((lc ^ swz<D>(rb)) * 16) + off_in);
  const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(pa);
  const bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(pb);
  return bf16x8{va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
}

// Writes a 32-row x D gradient held transposed in accumulators (lane = row, 16 d values
// per 32-wide block) as bf16 rows of `dst` (d contiguous), times `mul`.
template <int D>
__device__ __forceinline__ void store_rows(__bf16* dst, const f32x16 (&acc)[BwdCfg<D>::kDB], float mul, int lane) {
  const int hh = lane >> 5;
#pragma unroll
  for (int db = 0; db < BwdCfg<D>::kDB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 v4;
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] = (__bf16)(acc[db][4 * i + j] * mul);
      *reinterpret_cast<bf16x4*>(dst + 32 * db + 8 * i + 4 * hh) = v4;
    }
  }
}

// ---------------------------------------------------------------------------------------
// dQ: one workgroup (4 waves, 32 query rows each) per (batch, head, 128-row Q tile).  The
// four waves share every K/V stage: waves 0 and 1 load its two K pages, waves 2 and 3 its two
// V pages.  A wave whose 32 rows are all past the tile's valid rows keeps its loads and
// barriers and skips the products.
// A tile of at most 64 valid rows splits its keys instead: waves w and w + 2 hold the same 32
// rows (row group w & 1), wave w walks the even 32-key stages and wave w + 2 the odd ones,
// each into its own pair of stage buffers, and the two partial sums of dQ are added through
// LDS at the end.  Every wave then loads both the K and the V page of one page slot of its
// stage, so a tile of 33..64 rows keeps all four waves busy on half as many iterations.
// The two kinds of tile run as two launches (SPLIT): one kernel holding both walks needs
// more than 256 VGPRs.  The plan's device image lists the short tiles last.
template <int D, bool KPERM, bool SPLIT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) bwd_dq_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  // stage buffers as separate objects, so that the compiler can tell the loads into one
  // buffer from the reads of another and waits only for the stage it reads: K and V of the
  // two stages in flight (sk0/sv0, sk1/sv1), and for split tiles the odd stages' pair
  // (sk2/sv2, sk3/sv3), which also holds the partial sums of the final merge
  constexpr int kOdd = SPLIT ? C::kStage : 16;
  __shared__ __attribute__((aligned(1024))) uint8_t sk0[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sk1[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sv0[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sv1[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sk2[kOdd];
  __shared__ __attribute__((aligned(1024))) uint8_t sk3[kOdd];
  __shared__ __attribute__((aligned(1024))) uint8_t sv2[kOdd];
  __shared__ __attribute__((aligned(1024))) uint8_t sv3[kOdd];
  static_assert(C::kDB * 16 * 64 * 4 == 2 * C::kStage, "a wave's dQ accumulators fill two stage buffers");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5;
  const CONST_AS int32_t* pl_ent = (const CONST_AS int32_t*)p.pl_ent;
  const CONST_AS int32_t* pl_ptr = (const CONST_AS int32_t*)p.pl_ptr;
  const CONST_AS int32_t* tiles = (const CONST_AS int32_t*)p.dq_tiles;

  // this launch's tiles: the long ones first in the list, the short ones after them
  const int n_tiles = SPLIT ? p.n_dq_split : p.n_dq_tiles - p.n_dq_split;
  const int work = xcd_work(blockIdx.x, p.B * p.Hq * n_tiles);
  const int bh = work / n_tiles;
  const int t = work - bh * n_tiles + (SPLIT ? p.n_dq_tiles - p.n_dq_split : 0);
  const int b = bh / p.Hq, h = bh - b * p.Hq, g = h / p.grp;
  const int row0 = tiles[4 * t], rows = tiles[4 * t + 1], qblock = tiles[4 * t + 2];
  const int unit = (b * p.ub_mul) * p.sel_nh + h / p.uh_div;
  const int lrow = unit * p.nqb + qblock;
  const int e0 = pl_ptr[lrow], e1 = pl_ptr[lrow + 1];
  const int ns = (e1 - e0 + 1) >> 1;  // 32-key stages
  const int rg = SPLIT ? (wave & 1) : wave;  // row group
  const int kp = SPLIT ? (wave >> 1) : 0;    // split walk: even (0) or odd (1) stages

  // this lane's query: Q^T and dO^T B operands, its LSE (log2 units) and D
  const int qrow = rg * 32 + (lane & 31);
  const bool qvalid = qrow < rows;
  const bool active = rg * 32 < rows;  // the wave holds a valid row (uniform)
  const int qslot = row0 + (qvalid ? qrow : 0);
  const int qtok = p.qperm ? p.qperm[qslot] : qslot;
  bf16x8 qreg[C::kDS], goreg[C::kDS];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb + (int64_t)qtok * p.q_sn +
                       (int64_t)h * p.q_sh + hh * 8;
    const __bf16* gp = reinterpret_cast<const __bf16*>(p.dout) + (int64_t)b * p.o_sb + (int64_t)qtok * p.o_sn +
                       (int64_t)h * p.o_sh + hh * 8;
#pragma unroll
    for (int s = 0; s < C::kDS; ++s) {
      qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
      goreg[s] = *reinterpret_cast<const bf16x8*>(gp + 16 * s);
    }
  }
  const float lse = p.lse[(int64_t)bh * p.Nq + qtok];
  // a row without keys has LSE = -inf: +inf here makes every probability exp2(-inf) = 0
  const float lse2 = lse == kNegInf ? __builtin_huge_valf() : lse * kLog2e;
  const float dval = p.dvec[(int64_t)bh * p.Nq + qtok];
  // settled before the loop, so that no wait inside it has to cover them
  wait_vmcnt<0>();
  const int thr = p.causal ? causal_thr(p.q_pos0 + (int64_t)qtok) : 0x7ffffffe;

  const char* kslice = reinterpret_cast<const char*>(p.k) + ((int64_t)b * p.k_sb + (int64_t)g * p.k_sh) * 2;
  const char* vslice = reinterpret_cast<const char*>(p.v) + ((int64_t)b * p.v_sb + (int64_t)g * p.v_sh) * 2;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)kslice, (short)0, p.k_extent, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)vslice, (short)0, p.v_extent, 0x00020000);
  PageRows<D> pr;
  pr.init(lane);
  uint32_t tok[C::kInst];  // tokens of the next stage to fire
  int gst = 0;             // stage of the next gather
  auto gather = [&]() {
    const int e = e0 + 2 * gst + (wave & 1);  // entries past the list read as empty pages
    pr.template gather<KPERM>(e < e1 ? pl_ent[e] : 0, p.kperm, tok);
    ++gst;
  };
  auto fire = [&](uint8_t* kdst, uint8_t* vdst) __attribute__((always_inline)) {
    if (wave < 2)
      pr.fire1(tok, krsrc, p.k_sn_bytes, kdst, wave & 1);
    else
      pr.fire1(tok, vrsrc, p.v_sn_bytes, vdst, wave & 1);
  };
  // VMEM loads issued after a stage's page by the time its wait runs: the next stage's
  // page and, with a permutation, the gather of the stage after
  constexpr int kAfter = C::kInst + (KPERM ? C::kInst : 0);

  f32x16 dqacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) dqacc[db] = f32x16{};
  const float sl2 = p.scale_log2;

  // products of stage st (K and V pages in kb / vb) into dqacc
  auto compute = [&](int st, const uint8_t* kb, const uint8_t* vb) __attribute__((always_inline)) {
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
    for (int s = 0; s < C::kDS; ++s) {
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<D>(kb, lane, s), qreg[s], sacc, 0, 0, 0);
      dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<D>(vb, lane, s), goreg[s], dpacc, 0, 0, 0);
    }

    // register i holds key 8 (i / 4) + 4 hh + i % 4 of the stage: page i / 8, row key % 16
    const int ea = e0 + 2 * st;
    const int ent0 = pl_ent[ea];
    const int ent1 = ea + 1 < e1 ? pl_ent[ea + 1] : 0;
    // the products first, for every key: left to the compiler, the exponential would move
    // under the mask test below and each key would become a branch
    float dsv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dsv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], sl2, -lse2)) * (dpacc[i] - dval);
      pin(dsv[i]);
    }
    // mask: rows past the page's valid count, and keys after the query under a causal mask
    // (thr is INT_MAX - 1 without one); with permuted keys the causal test reads the key
    // tokens, in a pass of its own so that the plain case stays free of branches
    bf16x8 dsb[2];
    if (!p.causal && ent_nv(ent0) == 16 && ent_nv(ent1) == 16) {
      // two full pages and no causal mask (the common stage): nothing to mask
#pragma unroll
      for (int i = 0; i < 16; ++i) dsb[i >> 3][i & 7] = (__bf16)dsv[i];
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ent = (i >> 3) ? ent1 : ent0;
        const int rip = 8 * ((i >> 2) & 1) + 4 * hh + (i & 3);
        bool keep = rip < ent_nv(ent);
        if constexpr (!KPERM) keep = keep & (ent_slot(ent) + rip <= thr);
        dsb[i >> 3][i & 7] = (__bf16)(keep ? dsv[i] : 0.f);
      }
    }
    if constexpr (KPERM) {
      if (p.causal) {
        int ktok[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ent = (i >> 3) ? ent1 : ent0;
          const int rip = 8 * ((i >> 2) & 1) + 4 * hh + (i & 3);
          ktok[i] = p.kperm[ent_slot(ent) + (rip < ent_nv(ent) ? rip : 0)];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) dsb[i >> 3][i & 7] = ktok[i] > thr ? (__bf16)0.f : dsb[i >> 3][i & 7];
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
        dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(kb, lane, half, db), dsb[half], dqacc[db], 0, 0, 0);
  };

  // stage st: its K and V pages are in kb / vb; the next stage's go to kn / vn
  // (NEXT: a stage follows; known at compile time, so the steady state has no branch)
  auto stage = [&](auto next_tag, int st, const uint8_t* kb, const uint8_t* vb, uint8_t* kn, uint8_t* vn)
                   __attribute__((always_inline)) {
    if constexpr (decltype(next_tag)::value) {
      lds_barrier();  // both waves are done with the other buffer (stage st - 1)
      fire(kn, vn);   // stage st + 1
      gather();       // tokens of stage st + 2
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<kAfter>();  // stage st landed
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    if (active) compute(st, kb, vb);
    // each stage is scheduled on its own: no work moves between the two buffers' copies
    __builtin_amdgcn_sched_barrier(0);
  };

  // Split walk of a tile of at most 64 rows.  Iteration i covers stages 2i (KP = 0) and
  // 2i + 1 (KP = 1); the KP waves read buffer pair (ka, va) on even i and (kb, vb) on odd i,
  // and each wave loads page slot (wave & 1) of its stage of iteration i + 1, K and V, one
  // iteration ahead.  KP is a template argument, so that every buffer is a fixed LDS object.
  auto split_walk = [&](auto kp_tag) __attribute__((always_inline)) {
    constexpr int KP = decltype(kp_tag)::value;
    uint8_t* const ka = KP ? sk2 : sk0;
    uint8_t* const va = KP ? sv2 : sv0;
    uint8_t* const kb = KP ? sk3 : sk1;
    uint8_t* const vb = KP ? sv3 : sv1;
    const int npair = (ns + 1) >> 1;
    int gi = 0;  // iteration of the next gather
    auto sgather = [&]() {
      const int e = e0 + 2 * (2 * gi + KP) + (wave & 1);  // entries past the list read as empty pages
      pr.template gather<KPERM>(e < e1 ? pl_ent[e] : 0, p.kperm, tok);
      ++gi;
    };
    // VMEM loads issued after an iteration's pages by the time its wait runs: the next
    // iteration's K and V pages and, with a permutation, the gather of the one after
    constexpr int kAfterSplit = 2 * C::kInst + (KPERM ? C::kInst : 0);
    auto iter = [&](auto next_tag, int i, const uint8_t* kc, const uint8_t* vc, uint8_t* kn, uint8_t* vn)
                    __attribute__((always_inline)) {
      if constexpr (decltype(next_tag)::value) {
        lds_barrier();  // every wave is done with the other buffer pair (iteration i - 1)
        pr.fire1(tok, krsrc, p.k_sn_bytes, kn, wave & 1);  // iteration i + 1
        pr.fire1(tok, vrsrc, p.v_sn_bytes, vn, wave & 1);
        sgather();                                                                 // tokens of i + 2
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kAfterSplit>();  // iteration i landed
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();
      const int st = 2 * i + KP;
      if (active && st < ns) compute(st, kc, vc);
      __builtin_amdgcn_sched_barrier(0);
    };
    if (npair > 0) {
      sgather();
      pr.fire1(tok, krsrc, p.k_sn_bytes, ka, wave & 1);
      pr.fire1(tok, vrsrc, p.v_sn_bytes, va, wave & 1);
      sgather();
    }
    int i = 0;
    for (; i + 2 < npair; i += 2) {
      iter(BoolTag<true>{}, i, ka, va, kb, vb);
      iter(BoolTag<true>{}, i + 1, kb, vb, ka, va);
    }
    if (i + 1 < npair) {
      iter(BoolTag<true>{}, i, ka, va, kb, vb);
      iter(BoolTag<false>{}, i + 1, kb, vb, ka, va);
    } else if (i < npair) {
      iter(BoolTag<false>{}, i, ka, va, kb, vb);
    }
  };

  if constexpr (SPLIT) {
    if (kp == 0)
      split_walk(IntTag<0>{});
    else
      split_walk(IntTag<1>{});
    // merge: the odd-stage waves hand their partial sums to the even-stage waves of the same
    // rows through the odd buffers (row group 0 in sk2 / sk3, row group 1 in sv2 / sv3)
    __syncthreads();
    uint8_t* const r0 = rg ? sv2 : sk2;
    uint8_t* const r1 = rg ? sv3 : sk3;
    if (kp == 1 && active) {
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) {
        float* ob = reinterpret_cast<float*>((db < C::kDB / 2 ? r0 : r1)) + (db % (C::kDB / 2)) * 16 * 64;
#pragma unroll
        for (int e = 0; e < 16; ++e) ob[e * 64 + lane] = dqacc[db][e];
      }
    }
    __syncthreads();
    if (kp == 1 || !qvalid) return;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) {
      const float* ob = reinterpret_cast<const float*>((db < C::kDB / 2 ? r0 : r1)) + (db % (C::kDB / 2)) * 16 * 64;
#pragma unroll
      for (int e = 0; e < 16; ++e) dqacc[db][e] += ob[e * 64 + lane];
    }
  } else {
    if (ns > 0) {
      gather();
      fire(sk0, sv0);
      gather();
    }
    int st = 0;
    for (; st + 2 < ns; st += 2) {
      stage(BoolTag<true>{}, st, sk0, sv0, sk1, sv1);
      stage(BoolTag<true>{}, st + 1, sk1, sv1, sk0, sv0);
    }
    if (st + 1 < ns) {
      stage(BoolTag<true>{}, st, sk0, sv0, sk1, sv1);
      stage(BoolTag<false>{}, st + 1, sk1, sv1, sk0, sv0);
    } else if (st < ns) {
      stage(BoolTag<false>{}, st, sk0, sv0, sk1, sv1);
    }
    if (!qvalid) return;
  }

  __bf16* dst = reinterpret_cast<__bf16*>(p.dq) + (int64_t)b * p.q_sb + (int64_t)qtok * p.q_sn + (int64_t)h * p.q_sh;
  store_rows<D>(dst, dqacc, p.scale, lane);
}

// ---------------------------------------------------------------------------------------
// dK, dV: one workgroup (4 waves) per (batch, KV head, 64-row K tile); the query heads of
// the group are walked one after another, each over its unit's transposed page list.
// Waves 0 and 1 (score waves) hold K^T and V^T of keys 0..31 and 32..63 in registers and
// compute S and dP of each 32-query stage; they pass P^ and dS to LDS as bf16 B operands.
// Waves 2 and 3 (gradient waves) hold the dK^T and dV^T accumulators of the same keys and
// apply those operands one stage later.  Splitting the roles keeps every wave under 256
// VGPRs, so two workgroups share a CU (two waves per SIMD) and each wave's phase hides the
// other's latencies; the MFMA count per stage is the same as with one wave doing both.  The
// score and gradient waves of a key half with no valid key keep their loads and barriers
// and skip the products.
// Pipeline: score waves load the Q pages, gradient waves the dO pages and the row
// statistics (LSE, D and the causal bound of each query row: the score waves set the pace,
// the gradient waves have slack at the barrier), through registers, two stages ahead.  Q
// and dO have three stage buffers (the score waves read stage it while the gradient waves
// read stage it - 1 and stage it + 1 is written), the operands two.  One barrier per
// iteration, the same count in both roles.
template <int D, bool QPERM>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) bwd_dkdv_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t sq[3 * C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sg[3 * C::kStage];
  __shared__ __attribute__((aligned(16))) bf16x8 s_op[2][2][4][64];  // [stage & 1][key half][P^ 0, 1, dS 0, 1][lane]
  __shared__ __attribute__((aligned(16))) float s_lse[2][32];  // LSE in log2 units (+inf: no row)
  __shared__ __attribute__((aligned(16))) float s_d[2][32];
  __shared__ __attribute__((aligned(16))) int s_thr[2][32];    // causal bound of each query
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kh = wave & 1;     // key half; also the page of a stage this wave loads
  const bool score = wave < 2;  // score wave (loads Q) or gradient wave (loads dO)
  const int hh = lane >> 5;
  const CONST_AS int32_t* tpl_ptr = (const CONST_AS int32_t*)p.tpl_ptr;
  const CONST_AS int32_t* tiles = (const CONST_AS int32_t*)p.kv_tiles;

  const int work = xcd_work(blockIdx.x, p.B * p.Hkv * p.n_kv_tiles);
  const int bg = work / p.n_kv_tiles;
  const int t = work - bg * p.n_kv_tiles;
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int slot0 = tiles[4 * t], rows = tiles[4 * t + 1], kblock = tiles[4 * t + 2];

  // this lane's key
  const int krow = kh * 32 + (lane & 31);
  const bool kvalid = krow < rows;
  const bool active = kh * 32 < rows;  // the half holds a valid key (uniform)
  const int kslot = slot0 + (kvalid ? krow : 0);
  const int ktok = p.kperm ? p.kperm[kslot] : kslot;

  // stages: for each query head h of the group, ceil(pages / 2) stages of its list
  auto list_of = [&](int hi, int& a, int& z) {
    const int h = g * p.grp + hi;
    const int unit = (b * p.ub_mul) * p.sel_nh + h / p.uh_div;
    a = tpl_ptr[unit * p.nkb + kblock];
    z = tpl_ptr[unit * p.nkb + kblock + 1];
  };
  int nst = 0;
  for (int hi = 0; hi < p.grp; ++hi) {
    int a, z;
    list_of(hi, a, z);
    nst += (z - a + 1) >> 1;
  }
  const int n_it = nst > 0 ? nst + 1 : 0;  // the gradient waves run one stage behind
  // gather cursor: head index, next entry, end of its list (uniform); past the last list
  // it yields empty pages
  int c_h = 0, c_e = 0, c_z = 0;
  list_of(0, c_e, c_z);

  PageRows<D> pr;
  pr.init(lane);
  // the next stage to load: its head, this wave's page entry, the tokens of this lane's
  // load rows and the token of query row lane % 16 of the page (for the row statistics)
  int n_h = 0, n_ent = 0, n_stok = 0;
  uint32_t tok[C::kInst];
  // The raw entry of a stage is fetched one gather before it is used, with a vector load:
  // vector loads complete in order, so its use waits for it alone, while a scalar load can
  // only be waited for together with every LDS access in flight (and the next LDS wait
  // would take its whole latency).  Past its list the cursor reads entries it discards;
  // the entry array is followed by 64 zero words, so the load stays in bounds.
  const __amdgpu_buffer_rsrc_t ent_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.tpl_ent, (short)0, 0x7fffffff, 0x00020000);
  int f_h = 0;
  unsigned f_raw = 0;
  bool f_ok = false;
  auto fetch = [&]() {
    while (c_e >= c_z && c_h + 1 < p.grp) {
      ++c_h;
      list_of(c_h, c_e, c_z);
    }
    f_h = c_h;
    const int e = c_e + kh;
    f_ok = e < c_z;
    f_raw = __builtin_amdgcn_raw_buffer_load_b32(ent_rsrc, e * 4, 0, 0);
    c_e += 2;
  };
  auto gather = [&]() {
    n_h = f_h;
    n_ent = f_ok ? __builtin_amdgcn_readfirstlane((int)f_raw) : 0;
    pr.template gather<QPERM>(n_ent, p.qperm, tok);
    if (!score) {
      const int r = lane & 15;
      const int slot = ent_slot(n_ent) + (r < ent_nv(n_ent) ? r : 0);
      n_stok = QPERM ? p.qperm[slot] : slot;
    }
    __builtin_amdgcn_sched_barrier(0);
    fetch();  // the stage after
  };
  // the loaded page, not yet in LDS: Q (score waves) or dO (gradient waves) rows, and the
  // row statistics (gradient waves)
  u32x4 rr[C::kInst];
  float r_lse = 0.f, r_d = 0.f;
  int r_tok = 0, r_nv = 0;
  // buffer resources of the current head's Q (or dO) slice and LSE / D rows, rebuilt only
  // when the walk moves to the next head of the group (their 64-bit address arithmetic
  // would otherwise cost a few dozen scalar instructions per stage)
  int rs_h = -1;
  __amdgpu_buffer_rsrc_t t_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)p.q, (short)0, 0, 0x00020000);
  __amdgpu_buffer_rsrc_t lse_rsrc = t_rsrc, d_rsrc = t_rsrc;
  auto load = [&]() {
    if (n_h != rs_h) {
      rs_h = n_h;
      const int h = g * p.grp + n_h;
      if (score) {
        const char* qslice = reinterpret_cast<const char*>(p.q) + ((int64_t)b * p.q_sb + (int64_t)h * p.q_sh) * 2;
        t_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)qslice, (short)0, p.q_extent, 0x00020000);
      } else {
        const char* gslice = reinterpret_cast<const char*>(p.dout) + ((int64_t)b * p.o_sb + (int64_t)h * p.o_sh) * 2;
        t_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)gslice, (short)0, p.o_extent, 0x00020000);
        const int64_t srow = ((int64_t)b * p.Hq + h) * p.Nq;
        lse_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(p.lse + srow), (short)0, (uint32_t)p.Nq * 4u, 0x00020000);
        d_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(p.dvec + srow), (short)0, (uint32_t)p.Nq * 4u, 0x00020000);
      }
    }
    if (score) {
      pr.load(tok, t_rsrc, p.q_sn_bytes, rr);
    } else {
      pr.load(tok, t_rsrc, p.o_sn_bytes, rr);
      r_lse = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lse_rsrc, n_stok * 4, 0, 0));
      r_d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(d_rsrc, n_stok * 4, 0, 0));
      r_tok = n_stok;
      r_nv = ent_nv(n_ent);
    }
  };
  // page kh of stage buffer `buf`: rows 16 kh .. 16 kh + 15; lanes 0..15 of a gradient wave
  // write the statistics of those rows (for the score waves of the next iteration)
  auto store = [&](int buf, int sbuf) {
    pr.store(rr, (score ? sq : sg) + buf * C::kStage, kh, lane);
    if (!score && lane < 16) {
      const bool valid = lane < r_nv;
      s_lse[sbuf][16 * kh + lane] = (valid && r_lse != kNegInf) ? r_lse * kLog2e : __builtin_huge_valf();
      s_d[sbuf][16 * kh + lane] = valid ? r_d : 0.f;
      s_thr[sbuf][16 * kh + lane] = causal_thr(p.q_pos0 + (int64_t)r_tok);
    }
  };

  if (nst > 0) {
    fetch();
    gather();
    load();
    store(0, 0);
    gather();
    load();
    gather();
  }

  if (score) {
    // K^T and V^T B operands of this lane's key
    bf16x8 kreg[C::kDS], vreg[C::kDS];
    {
      const __bf16* kp = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb + (int64_t)ktok * p.k_sn +
                         (int64_t)g * p.k_sh + hh * 8;
      const __bf16* vp = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.v_sb + (int64_t)ktok * p.v_sn +
                         (int64_t)g * p.v_sh + hh * 8;
#pragma unroll
      for (int s = 0; s < C::kDS; ++s) {
        kreg[s] = *reinterpret_cast<const bf16x8*>(kp + 16 * s);
        vreg[s] = *reinterpret_cast<const bf16x8*>(vp + 16 * s);
      }
    }
    // settle these loads here: left in flight into the loop, they would make the loop's
    // first use of them wait for every load outstanding there, prefetches included
    wait_vmcnt<0>();
    const float sl2 = p.scale_log2;
    // per-lane byte offset of the A operand of k-step s inside a stage buffer (row lane % 32,
    // logical chunk 2s + hh); the buffer itself is a compile-time offset (the loop below is
    // unrolled over the three buffers), so no operand read needs an address instruction
    uint32_t roff[C::kDS];
    {
      const int r = lane & 31;
#pragma unroll
      for (int s = 0; s < C::kDS; ++s) roff[s] = r * C::kRowBytes + (((2 * s + hh) ^ swz<D>(r)) * 16);
    }
    // iteration it with stage it in buffer B (compile-time)
    auto iter = [&](auto buf_tag, int it) __attribute__((always_inline)) {
      constexpr int B = decltype(buf_tag)::value;
      lds_barrier();  // stage it is in LDS; everybody is done with the buffers written next
      if (it + 1 < nst) {
        store((B + 1) % 3, (it + 1) & 1);  // stage it + 1
        load();                            // stage it + 2
        gather();                          // tokens of stage it + 3
      }
      if (it < nst && active) {
        const uint8_t* qb = sq + B * C::kStage;
        const uint8_t* gb = sg + B * C::kStage;
        f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
        for (int s = 0; s < C::kDS; ++s) {
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(qb + roff[s]), kreg[s], sacc, 0, 0, 0);
          dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(gb + roff[s]), vreg[s], dpacc, 0, 0, 0);
        }
        // register i holds query 8 (i / 4) + 4 hh + i % 4 of the stage and this lane's key
        const int sb = it & 1;
        float pv[16], dv[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 l4 = *reinterpret_cast<const float4*>(&s_lse[sb][8 * j + 4 * hh]);
          const float4 d4 = *reinterpret_cast<const float4*>(&s_d[sb][8 * j + 4 * hh]);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pv[4 * j + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * j + e], sl2, -lv[e]));
            dv[4 * j + e] = dd[e];
          }
        }
        // causal mask: a key after the query contributes nothing (without the mask, every
        // key of a listed page row is kept; rows past a page's end already have P^ = 0)
        if (p.causal) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int4 t4 = *reinterpret_cast<const int4*>(&s_thr[sb][8 * j + 4 * hh]);
            const int tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) pv[4 * j + e] = ktok <= tv[e] ? pv[4 * j + e] : 0.f;
          }
        }
        bf16x8 pb[2], dsb[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pb[i >> 3][i & 7] = (__bf16)pv[i];
          dsb[i >> 3][i & 7] = (__bf16)(pv[i] * (dpacc[i] - dv[i]));
        }
        s_op[sb][kh][0][lane] = pb[0];
        s_op[sb][kh][1][lane] = pb[1];
        s_op[sb][kh][2][lane] = dsb[0];
        s_op[sb][kh][3][lane] = dsb[1];
      }
    };
    for (int it = 0; it < n_it; it += 3) {
      iter(IntTag<0>{}, it);
      if (it + 1 < n_it) iter(IntTag<1>{}, it + 1);
      if (it + 2 < n_it) iter(IntTag<2>{}, it + 2);
    }
    return;
  }

  f32x16 dkacc[C::kDB], dvacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }
  int cur = 0;
  for (int it = 0; it < n_it; ++it) {
    lds_barrier();  // matches the score waves' barrier of the same iteration
    if (it + 1 < nst) {
      store(cur == 2 ? 0 : cur + 1, (it + 1) & 1);
      load();
      gather();
    }
    if (it >= 1 && active) {  // stage it - 1
      const int pb_ = cur == 0 ? 2 : cur - 1;
      const uint8_t* qb = sq + pb_ * C::kStage;
      const uint8_t* gb = sg + pb_ * C::kStage;
      const int sb = (it - 1) & 1;
      bf16x8 pb[2], dsb[2];
      pb[0] = s_op[sb][kh][0][lane];
      pb[1] = s_op[sb][kh][1][lane];
      dsb[0] = s_op[sb][kh][2][lane];
      dsb[1] = s_op[sb][kh][3][lane];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) {
          dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(gb, lane, half, db), pb[half], dvacc[db], 0, 0, 0);
          dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(qb, lane, half, db), dsb[half], dkacc[db], 0, 0, 0);
        }
    }
    cur = cur == 2 ? 0 : cur + 1;
  }

  if (!kvalid) return;
  __bf16* dkp = reinterpret_cast<__bf16*>(p.dk) + (int64_t)b * p.k_sb + (int64_t)ktok * p.k_sn + (int64_t)g * p.k_sh;
  __bf16* dvp = reinterpret_cast<__bf16*>(p.dv) + (int64_t)b * p.v_sb + (int64_t)ktok * p.v_sn + (int64_t)g * p.v_sh;
  store_rows<D>(dkp, dkacc, p.scale, lane);
  store_rows<D>(dvp, dvacc, 1.f, lane);
}

// ---------------------------------------------------------------------------------------
template <int D>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  const int64_t nrows = (int64_t)p.B * p.Hq * p.Nq;
  if (nrows > 0) {
    constexpr int kRowsPerBlock = 4 * (64 / (D / 8));
    hipLaunchKernelGGL((bwd_dot_kernel<D>), dim3((unsigned)((nrows + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(256),
                       0, stream, p);
  }
  const int64_t n_kv = (int64_t)p.B * p.Hkv * p.n_kv_tiles;
  if (n_kv > 0) {
    if (p.qperm)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3((unsigned)n_kv), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3((unsigned)n_kv), dim3(256), 0, stream, p);
  }
  // dQ: the tiles of more than kDqSplitRows rows, then the short tiles with the key split
  const int64_t n_long = (int64_t)p.B * p.Hq * (p.n_dq_tiles - p.n_dq_split);
  const int64_t n_short = (int64_t)p.B * p.Hq * p.n_dq_split;
  if (n_long > 0) {
    if (p.kperm)
      hipLaunchKernelGGL((bwd_dq_kernel<D, true, false>), dim3((unsigned)n_long), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, false, false>), dim3((unsigned)n_long), dim3(256), 0, stream, p);
  }
  if (n_short > 0) {
    if (p.kperm)
      hipLaunchKernelGGL((bwd_dq_kernel<D, true, true>), dim3((unsigned)n_short), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, false, true>), dim3((unsigned)n_short), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int d, hipStream_t stream) {
  return d == 128 ? launch_bwd_d<128>(p, stream) : launch_bwd_d<64>(p, stream);
}

}  // namespace bsattn
