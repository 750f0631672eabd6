// Exact block-sparse attention forward for gfx950 (MI355X).
//
// A Q tile of one (batch, head) walks its page list: every entry is a 16-row K/V page of
// one block, so the stages loaded into LDS pack pages of several logical blocks (KPage
// abstract, zhuanzhiai page 1, sentence 2).  Pages are gathered from HBM straight into LDS
// (global_load_lds, 16 bytes per lane): nothing compacted is ever written back.  Q tiles
// come in two shapes (sentence 3): 128 rows x 128-key K tiles and 64 rows x 256-key K
// tiles.  Exact masking (sentence 4) clears empty page slots and, for causal problems, keys
// after the query.
//
// The main path is the ping-pong walk further down (both shapes, one launch).  The 4-wave
// kernel right below serves the problems the walk does not take (permuted keys under a
// causal mask): per wave and K tile it does 32 queries x 64 keys --
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q^T in registers;
//                  the accumulator gives each lane one query (lane % 32) and 64 keys.
//   online softmax in fp32 (row max / sum per lane, one cross-half exchange),
//                  exp2 with log2(e) folded into the scale.
//   O^T += V^T P^T A = V^T read from LDS with ds_read_b64_tr_b16, B = P^T straight from
//                  the score accumulators converted to bf16; the O^T accumulator again
//                  gives each lane one query, so rescaling and the epilogue stay in-lane.
// The exponentials of one 32-key block are followed by that block's P.V products, so the
// matrix cores work while the next block's exponentials are computed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "device_common.hpp"
#include "kernel_params.hpp"

namespace bsattn {

template <int D, int NRG, int NKG, int KB>
struct Cfg {
  static constexpr int kTileK = 32 * KB * NKG;       // keys per pipeline stage (LDS tile)
  static constexpr int kPPT = kTileK / 16;           // pages per stage
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;              // 16-byte chunks per row
  static constexpr int kRowsPerInst = 64 / kChunks;  // rows per 64-lane 16-byte load
  static constexpr int kRowsPerWave = kTileK / 4;
  static constexpr int kWavePages = kRowsPerWave / 16;
  static constexpr int kInst = kRowsPerWave / kRowsPerInst;  // loads per wave per tensor
  static constexpr int kBufBytes = kTileK * kRowBytes;
  static constexpr int kDS = D / 16;                 // k-steps of QK^T
  static constexpr int kDB = D / 32;                 // 32-wide d blocks of O^T
  // two workgroups per CU when the LDS allows it (three waves per SIMD would leave 168
  // VGPRs: too few)
  static constexpr int kLds = 2 * kBufBytes + kTileK * 4;
  static constexpr int kWavesPerEU = 2 * kLds <= 160 * 1024 ? 2 : 1;
};

template <int D, int NRG, int NKG, int KB, bool KPERM>
__global__ void __launch_bounds__(256)
    __attribute__((amdgpu_waves_per_eu(Cfg<D, NRG, NKG, KB>::kWavesPerEU, Cfg<D, NRG, NKG, KB>::kWavesPerEU)))
    fwd_kernel(FwdParams p) {
  using C = Cfg<D, NRG, NKG, KB>;
  // K and V tiles as separate objects: the compiler can then tell that reads of one never
  // touch the other's in-flight loads and adds no waits of its own.  After the last tile the
  // two arrays hold the key-group merge (row group 0 in K, row group 1 in V).
  __shared__ __attribute__((aligned(1024))) uint8_t smem_k[C::kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t smem_v[C::kBufBytes];
  static_assert(NKG == 1 || (NRG <= 2 && (C::kDB * 16 + 2) * 64 * 4 <= C::kBufBytes), "merge buffer fits");
  __shared__ int ktok_lds[KPERM ? C::kTileK : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % NRG;
  const int kg = wave / NRG;
  const int hh = lane >> 5;

  // plan tables are read-only during the kernel: constant address space -> scalar loads
  const CONST_AS int32_t* pl_ent = (const CONST_AS int32_t*)p.pl_ent;
  const CONST_AS int32_t* pl_ptr = (const CONST_AS int32_t*)p.pl_ptr;
  const CONST_AS int32_t* qtiles = (const CONST_AS int32_t*)p.qtiles;  // QTileDev records

  // ---- work item (XCD-aware: consecutive items share an XCD's L2) ----
  int work;
  {
    const int n = p.n_work, blk = blockIdx.x;
    const int x = blk & 7, i = blk >> 3, q = n >> 3, r = n & 7;
    work = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
  }
  const int bh = work / p.n_qtiles;
  const int t = work - bh * p.n_qtiles;
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int g = h / p.grp;
  struct {
    int row0, rows, qblock;
  } qt;
  static_assert(sizeof(QTileDev) == 4 * sizeof(int32_t), "QTileDev layout");
  qt.row0 = qtiles[4 * t];
  qt.rows = qtiles[4 * t + 1];
  qt.qblock = qtiles[4 * t + 2];
  const int unit = (b * p.ub_mul) * p.sel_nh + h / p.uh_div;
  const int row = unit * p.nqb + qt.qblock;
  const int e0 = pl_ptr[row];
  const int e1 = pl_ptr[row + 1];
  const int nkt = (e1 - e0 + C::kPPT - 1) / C::kPPT;

  // ---- Q^T operand: lane holds query (lane % 32) of its row group, 8 d per k-step ----
  const int qrow = rg * 32 + (lane & 31);
  const bool qvalid = qrow < qt.rows;
  const int qslot = qt.row0 + (qvalid ? qrow : 0);
  const int qtok = p.qperm ? p.qperm[qslot] : qslot;
  bf16x8 qreg[C::kDS];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb + (int64_t)qtok * p.q_sn +
                       (int64_t)h * p.q_sh + hh * 8;
#pragma unroll
    for (int s = 0; s < C::kDS; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }
  // causal threshold for this lane's query: a key is kept iff its token <= thr
  int thr = 0x7ffffffe;
  if (p.causal) {
    const int64_t qp = p.q_pos0 + (int64_t)qtok;
    thr = qp < -1 ? -1 : (qp > 0x7ffffffe ? 0x7ffffffe : (int)qp);
  }
  const int64_t minq_pos = p.q_pos0 + qt.row0 + rg * 32;  // smallest query position of the wave (identity Q layout)

  // ---- loader: K/V pages -> LDS with buffer loads (SGPR base + 32-bit offsets) ----
  // Row r of the tile goes to LDS row r; lane (ld_lr, ld_pc) of a load fills physical chunk
  // ld_pc of row r, i.e. logical chunk ld_pc ^ swz(r).  The row's page is uniform per load.
  const int ld_lr = lane / C::kChunks;  // row inside one load
  const int ld_pc = lane % C::kChunks;  // physical chunk slot this lane fills
  constexpr int kPeriod = 16 / C::kRowsPerInst;  // loads per 16-row page
  const char* kslice = reinterpret_cast<const char*>(p.k) + ((int64_t)b * p.k_sb + (int64_t)g * p.k_sh) * 2;
  const char* vslice = reinterpret_cast<const char*>(p.v) + ((int64_t)b * p.v_sb + (int64_t)g * p.v_sh) * 2;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)kslice, (short)0, p.k_extent, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)vslice, (short)0, p.v_extent, 0x00020000);
  int ld_rip[kPeriod], ld_cb[kPeriod];     // row inside the page, logical chunk byte offset
  uint32_t ld_vk[kPeriod], ld_vv[kPeriod];  // per-lane K / V byte offsets of a full page's rows
#pragma unroll
  for (int n = 0; n < kPeriod; ++n) {
    ld_rip[n] = (n * C::kRowsPerInst + ld_lr) & 15;
    ld_cb[n] = (ld_pc ^ swz<D>(ld_rip[n])) * 16;
    ld_vk[n] = (uint32_t)ld_rip[n] * p.k_sn_bytes + ld_cb[n];
    ld_vv[n] = (uint32_t)ld_rip[n] * p.v_sn_bytes + ld_cb[n];
  }
  int ents[C::kWavePages];          // page entries of this wave's load rows (uniform)
  bool ents_full = true;            // all of them are full 16-row pages (uniform)
  int ldtok[KPERM ? C::kInst : 1];  // gathered key tokens (K permutation only)
  int ment[2 * KB];                 // page entries of this wave's key slice (uniform)

  // Page entries (and, with a K permutation, tokens) of the rows this wave loads for K tile
  // kt, and whether this wave's 128-key slice of that tile needs masking: a partial or empty
  // page slot, or (causal) keys that may follow one of the wave's queries.  With a K
  // permutation the slice's tokens also go to ktok_lds (empty slots INT_MAX).
  auto fetch_tokens = [&](int kt) -> bool {
    // two scalar vector loads: the wave's load pages and its key slice (the entry array is
    // zero-padded, so reading past a list's end stays in bounds; those slots count as empty)
    const int etile = e0 + kt * C::kPPT;
    const int el = etile + wave * C::kWavePages;
    const int es = etile + kg * 2 * KB;
    const SVec<C::kWavePages> lv = *(const CONST_AS SVec<C::kWavePages>*)(pl_ent + el);
    const SVec<2 * KB> sv = *(const CONST_AS SVec<2 * KB>*)(pl_ent + es);
    ents_full = true;
#pragma unroll
    for (int pp = 0; pp < C::kWavePages; ++pp) {
      ents[pp] = el + pp < e1 ? lv[pp] : 0;
      ents_full &= (ents[pp] & 31) == 16;
    }
    if constexpr (KPERM) {
#pragma unroll
      for (int n = 0; n < C::kInst; ++n) {
        const int ent = ents[(n * C::kRowsPerInst) >> 4];
        const int nv = ent & 31, rip = ld_rip[n % kPeriod];
        const int tok = p.kperm[ent_slot(ent) + (rip < nv ? rip : 0)];
        ldtok[n] = tok;
        if (ld_pc == 0) ktok_lds[wave * C::kRowsPerWave + n * C::kRowsPerInst + ld_lr] = rip < nv ? tok : 0x7fffffff;
      }
    }
    bool need = false;
    int maxkey = -1;
#pragma unroll
    for (int pp = 0; pp < 2 * KB; ++pp) {
      ment[pp] = es + pp < e1 ? sv[pp] : 0;
      const int nv = ment[pp] & 31;
      need |= nv < 16;
      const int last = ent_slot(ment[pp]) + nv - 1;
      maxkey = (nv > 0 && last > maxkey) ? last : maxkey;
    }
    if (p.causal) {
      if (KPERM || p.qperm)
        need = true;
      else
        need |= (int64_t)maxkey > minq_pos;
    }
    return need;
  };
  // Loads of one tensor's rows for the tile whose entries fetch_tokens read.  Rows past a
  // page's valid count (and empty page slots) load the page's first row / token 0: finite
  // data that the mask removes.  Only the per-lane offsets depend on whether every page is
  // full; the loads themselves are issued unconditionally, so the compiler can count them.
  auto issue = [&](const __amdgpu_buffer_rsrc_t& rsrc, uint32_t sn_bytes, const uint32_t (&vfull)[kPeriod],
                   uint8_t* buf) {
    uint32_t voff[C::kInst], soff[C::kInst];
#pragma unroll
    for (int n = 0; n < C::kInst; ++n) {
      if constexpr (KPERM) {
        voff[n] = (uint32_t)ldtok[n] * sn_bytes + ld_cb[n % kPeriod];
        soff[n] = 0;
      } else {
        const int ent = ents[(n * C::kRowsPerInst) >> 4];
        voff[n] = vfull[n % kPeriod];
        if (!ents_full && ld_rip[n % kPeriod] >= (ent & 31)) voff[n] = (uint32_t)ld_cb[n % kPeriod];
        soff[n] = (uint32_t)ent_slot(ent) * sn_bytes;
      }
    }
#pragma unroll
    for (int n = 0; n < C::kInst; ++n) {
      uint8_t* dst = buf + (wave * C::kRowsPerWave + n * C::kRowsPerInst) * C::kRowBytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)dst, 16, (int)voff[n], (int)soff[n], 0, 0);
    }
  };

  // ---- running softmax state and O^T accumulators ----
  float m_run = kNegInf;
  float l_run = 0.f;
  f32x16 oacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) oacc[db] = f32x16{};

  const float sl2 = p.scale_log2;
  const int kbase_row = kg * 32 * KB;
  // per-lane constants of the transposed V reads
  const int v_rr = (lane & 15) >> 2, v_qq = lane & 3, v_dsub = (lane >> 4) & 1;

  bool nm_next = false;
  if (nkt > 0) {
    nm_next = fetch_tokens(0);
    issue(krsrc, p.k_sn_bytes, ld_vk, smem_k);
    issue(vrsrc, p.v_sn_bytes, ld_vv, smem_v);
  }

  // One K tile.  MORE: a next tile exists and its loads are issued here.  The last tile is
  // a separate instantiation so that, inside the loop, the loads are unconditional: the
  // compiler then sees that the K tile at the loop head is older than the V tile behind it
  // and waits for the K loads only, instead of for every load in flight.
  auto tile = [&](int kt, auto more_tag) __attribute__((always_inline)) {
    constexpr bool MORE = decltype(more_tag)::value;
    const bool need_mask = nm_next;

    wait_vmcnt<C::kInst>();  // K tile landed (V may still be in flight)
    lds_barrier();

    // ---- S^T = K Q^T ----
    f32x16 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int s = 0; s < C::kDS; ++s) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int r = kbase_row + 32 * kb + (lane & 31);
        const int c = (2 * s + hh) ^ swz<D>(r);
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(smem_k + r * C::kRowBytes + c * 16);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[kb], 0, 0, 0);
      }
    }

    // ---- exact mask: empty page slots, causally hidden keys ----
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (KPERM) {
            const i32x4 t4 = *reinterpret_cast<const i32x4*>(&ktok_lds[kbase_row + 32 * kb + 8 * i + 4 * hh]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (t4[j] > thr) sacc[kb][4 * i + j] = kNegInf;
          } else {
            // key 32kb + 8i + 4hh + j is row 8(i&1) + 4hh + j of page 2kb + i/2
            const int ent = ment[2 * kb + (i >> 1)];
            int lim = (ent & 31) - 1;
            if (p.causal) lim = min(lim, thr - ent_slot(ent));
            const int rip0 = 8 * (i & 1) + 4 * hh;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (rip0 + j > lim) sacc[kb][4 * i + j] = kNegInf;
          }
        }
      }
    }

    // ---- online softmax: tile max, rescale ----
    float mt = fmaxf(max16(sacc[0]), max16(sacc[1]));
    if constexpr (KB == 4) mt = fmaxf(mt, fmaxf(max16(sacc[2]), max16(sacc[3])));
    mt = xor32_max(mt);
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * sl2);
    const float nb = -m_use * sl2;
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) oacc[db] *= alpha;
    }
    l_run *= alpha;

    wait_vmcnt<0>();  // V tile landed
    lds_barrier();    // every wave is done with the K buffer and the token list
    if constexpr (MORE) {
      nm_next = fetch_tokens(kt + 1);
      issue(krsrc, p.k_sn_bytes, ld_vk, smem_k);
    }

    // ---- per 32-key block: P = exp2(S*c - m*c), then O^T += V^T P^T ----
    float lsum[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      bf16x8 pb[2];
      float pe[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][e], sl2, nb));
        pb[e >> 3][e & 7] = (__bf16)pe[e];
      }
      lsum[kb] = sum16(pe);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int key_a = kbase_row + 32 * kb + 16 * half + 4 * hh + v_rr;
        const int key_b = key_a + 8;
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) {
          const int lc = 4 * db + 2 * v_dsub + (v_qq >> 1);
          const int off_in = (v_qq & 1) * 8;
          LDS_AS bf16x4* pa = (LDS_AS bf16x4*)(smem_v + key_a * C::kRowBytes + ((lc ^ swz<D>(key_a)) * 16) + off_in);
          LDS_AS bf16x4* pv = (LDS_AS bf16x4*)(smem_v + key_b * C::kRowBytes + ((lc ^ swz<D>(key_b)) * 16) + off_in);
          const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(pa);
          const bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(pv);
          const bf16x8 av = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[half], oacc[db], 0, 0, 0);
        }
      }
    }

    if constexpr (KB == 4)
      l_run += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    else
      l_run += lsum[0] + lsum[1];

    if constexpr (MORE) {
      lds_barrier();  // every wave is done with the V buffer
      issue(vrsrc, p.v_sn_bytes, ld_vv, smem_v);
    }
  };
  for (int kt = 0; kt + 1 < nkt; ++kt) tile(kt, BoolTag<true>{});
  if (nkt > 0) tile(nkt - 1, BoolTag<false>{});

  // ---- finish: combine lane halves, merge key groups, write O and LSE ----
  float l_tot = xor32_sum(l_run);
  float m_fin = m_run;
  if constexpr (NKG == 2) {
    // key group 1 hands (m, l, O^T) to key group 0 through LDS (the K buffer is free)
    __syncthreads();
    float* mb = reinterpret_cast<float*>(rg == 0 ? smem_k : smem_v);
    if (kg == 1) {
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) mb[(db * 16 + e) * 64 + lane] = oacc[db][e];
      mb[(C::kDB * 16) * 64 + lane] = m_run;
      mb[(C::kDB * 16 + 1) * 64 + lane] = l_tot;
    }
    __syncthreads();
    if (kg == 1) return;
    const float m1 = mb[(C::kDB * 16) * 64 + lane];
    const float l1 = mb[(C::kDB * 16 + 1) * 64 + lane];
    const float mm = fmaxf(m_run, m1);
    const float mu = (mm == kNegInf) ? 0.f : mm;
    const float a0 = __builtin_amdgcn_exp2f((m_run - mu) * sl2);
    const float a1 = __builtin_amdgcn_exp2f((m1 - mu) * sl2);
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] = oacc[db][e] * a0 + mb[(db * 16 + e) * 64 + lane] * a1;
    l_tot = l_tot * a0 + l1 * a1;
    m_fin = mm;
  }

  if (!qvalid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  __bf16* op = reinterpret_cast<__bf16*>(p.o) + (int64_t)b * p.o_sb + (int64_t)qtok * p.o_sn + (int64_t)h * p.o_sh;
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 v4;
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] = (__bf16)(oacc[db][4 * i + j] * inv);
      *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * i + 4 * hh) = v4;
    }
  }
  if (hh == 0) {
    const float lse = l_tot > 0.f ? m_fin * p.scale + __logf(l_tot) : kNegInf;
    p.lse[((int64_t)b * p.Hq + h) * p.Nq + qtok] = lse;
  }
}

// ---------------------------------------------------------------------------------------
// Ping-pong walk: 8 waves, two per SIMD.  Waves 0-3 (group 0) and 4-7 (group 1) split the
// tile's 64-key stages (4 pages): group g takes stages g, g + 2, g + 4, ...  The walk
// alternates two kinds of phase between workgroup barriers: a matrix phase (P.V of the
// group's previous stage, then S^T = K Q^T of its current one) and a vector phase (mask,
// online softmax and exponentials of the current stage).  Group 1 runs one phase behind
// group 0, so in every phase each SIMD holds one wave issuing MFMAs and one issuing vector
// instructions, and the two execute side by side.  The P.V products read their V^T operands
// straight from the V stage with transposing LDS reads (two per operand).  K and V stages
// are double-buffered per group: the matrix phase issues the next stage's K pages, the
// vector phase (which no longer touches LDS) the next stage's V pages.
//
// The two Q-tile shapes of the plan (KPage abstract, zhuanzhiai page 1, sentence 3) differ
// only in how a group's four waves share a stage:
//   128-row tiles: wave w of a group holds row group w (32 queries) and all 64 keys of the
//                  stage (two 32-key blocks): 32 MFMAs per wave and matrix phase at d = 128;
//   64-row tiles:  wave w holds row group w & 1 and the 32-key half w >> 1 of the stage:
//                  16 MFMAs per matrix phase.  Four consecutive stages are one 256-key K
//                  tile of the plan; two groups x two slots keep all four in LDS at once.
// Each (group, key half) keeps its own softmax state over its keys; the states of a row
// group are merged through LDS at the end.  The waves of a row group that holds only
// padding (rows past the tile's valid count) walk a copy of the loop without products and
// exponentials: they keep their share of the loads and every barrier.
// The branch is taken once per tile, so the busy waves run branch-free phases.  Both shapes
// use the same LDS stage layout, so one launch can run tiles of both kinds.
//
// The softmax reference max is lazy: it moves only when a stage's max exceeds it by more
// than 2^8 in exp2 units, so O is rescaled a few times per tile instead of at most stages.
// Probabilities are then bounded by 2^8 instead of 1, which fp32 sums and bf16 operands hold
// with the same relative precision; the result is the same softmax.
template <int D>
struct PPCfg {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;               // 16-byte chunks per row
  static constexpr int kRowsPerInst = 64 / kChunks;   // rows per 64-lane 16-byte load
  static constexpr int kInst = 16 / kRowsPerInst;     // loads per wave per tensor per stage (one page)
  static constexpr int kStage = 64 * kRowBytes;       // one 64-key stage of K or V
  static constexpr int kDS = D / 16;                  // k-steps of QK^T
  static constexpr int kDB = D / 32;                  // 32-wide d blocks of O^T
  // a wave's end state for the merge: O^T accumulators (kDB x 16 floats per lane), and
  // max and sum of up to six records (64 lanes each)
  static constexpr int kRecord = kDB * 16 * 64 * 4;
  static constexpr int kMlBytes = 6 * 2 * 64 * 4;
};

constexpr float kLazySlack = 8.f;  // log2 units the reference max may trail the true max

// LDS of the walk: stage buffers by slot (group g's stage at offset g * kStage of each
// array) and the max / sum records of the final merge.  Separate objects, so the compiler
// can tell reads of one from loads into another.
template <int D>
struct PPSmem {
  uint8_t* sk0;
  uint8_t* sk1;
  uint8_t* sv0;
  uint8_t* sv1;
  uint8_t* sml;
};

// One Q tile (work item `work` of the tiles at qtiles) walked by the workgroup.  R64: the
// tile is a 64-row tile (see above).
template <int D, bool KPERM, bool R64>
__device__ __forceinline__ void pp_walk(const FwdParams& p, const CONST_AS int32_t* qtiles, int n_qtiles, int work,
                                        const PPSmem<D>& sm) {
  using C = PPCfg<D>;
  constexpr int JB = R64 ? 1 : 2;  // 32-key blocks of a stage per wave
  uint8_t* const sk0 = sm.sk0;
  uint8_t* const sk1 = sm.sk1;
  uint8_t* const sv0 = sm.sv0;
  uint8_t* const sv1 = sm.sv1;
  uint8_t* const sml = sm.sml;
  static_assert(2 * C::kRecord <= 2 * C::kStage, "two O^T records fit in a stage slot array");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                  // stage group
  const int wr = wave & 3;                    // the page of each stage this wave loads
  const int rg = R64 ? (wr & 1) : wr;         // row group
  const int kh = R64 ? (wr >> 1) : 0;         // key half of the stage (64-row tiles)
  const int hh = lane >> 5;

  const CONST_AS int32_t* pl_ent = (const CONST_AS int32_t*)p.pl_ent;
  const CONST_AS int32_t* pl_ptr = (const CONST_AS int32_t*)p.pl_ptr;
  const CONST_AS int32_t* kperm = (const CONST_AS int32_t*)p.kperm;

  const int bh = work / n_qtiles;
  const int t = work - bh * n_qtiles;
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int g = h / p.grp;
  const int qt_row0 = qtiles[4 * t], qt_rows = qtiles[4 * t + 1], qt_qblock = qtiles[4 * t + 2];
  const int unit = (b * p.ub_mul) * p.sel_nh + h / p.uh_div;
  const int row = unit * p.nqb + qt_qblock;
  const int e0 = pl_ptr[row];
  const int e1 = pl_ptr[row + 1];
  const int ns = (e1 - e0 + 3) >> 2;        // 64-key stages
  const int my_n = (ns + 1 - grp) >> 1;     // this group's stages: global 2j + grp, j < my_n
  // a row group past the tile's valid rows holds only padding: no products for it (uniform)
  const bool active = rg * 32 < qt_rows;

  // ---- Q^T operand: lane holds query (lane % 32) of its row group, 8 d per k-step ----
  const int qrow = rg * 32 + (lane & 31);
  const bool qvalid = qrow < qt_rows;
  const int qslot = qt_row0 + (qvalid ? qrow : 0);
  const int qtok = p.qperm ? p.qperm[qslot] : qslot;
  bf16x8 qreg[C::kDS];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb + (int64_t)qtok * p.q_sn +
                       (int64_t)h * p.q_sh + hh * 8;
#pragma unroll
    for (int s = 0; s < C::kDS; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }
  int thr = 0x7ffffffe;  // causal: a key is kept iff its token <= thr
  if (p.causal) {
    const int64_t qp = p.q_pos0 + (int64_t)qtok;
    thr = qp < -1 ? -1 : (qp > 0x7ffffffe ? 0x7ffffffe : (int)qp);
  }
  const int64_t minq_pos = p.q_pos0 + qt_row0 + rg * 32;  // smallest query position of the wave (identity Q)

  // ---- loader: page wr of a stage -> rows wr * 16 .. + 15 of the group's stage buffer ----
  const int ld_lr = lane / C::kChunks;
  const int ld_pc = lane % C::kChunks;
  const char* kslice = reinterpret_cast<const char*>(p.k) + ((int64_t)b * p.k_sb + (int64_t)g * p.k_sh) * 2;
  const char* vslice = reinterpret_cast<const char*>(p.v) + ((int64_t)b * p.v_sb + (int64_t)g * p.v_sh) * 2;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)kslice, (short)0, p.k_extent, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)vslice, (short)0, p.v_extent, 0x00020000);
  int ld_rip[C::kInst], ld_cb[C::kInst];
  uint32_t ld_vk[C::kInst], ld_vv[C::kInst];
#pragma unroll
  for (int n = 0; n < C::kInst; ++n) {
    ld_rip[n] = n * C::kRowsPerInst + ld_lr;  // row inside the page
    ld_cb[n] = (ld_pc ^ swz<D>(ld_rip[n])) * 16;
    ld_vk[n] = (uint32_t)ld_rip[n] * p.k_sn_bytes + ld_cb[n];
    ld_vv[n] = (uint32_t)ld_rip[n] * p.v_sn_bytes + ld_cb[n];
  }
  const int goff = grp * C::kStage;                      // this group's stage in a slot array
  const int woff = goff + wr * 16 * C::kRowBytes;        // this wave's page in it

  // The four page entries of local stage j (global 2j + grp), zero past the list (the entry
  // array is zero-padded past its end, so the scalar load stays in bounds).  They are loaded
  // two phases ahead of their first use and kept in scalar registers.
  // The raw words are only checked against the list's end where they are used, so that no
  // instruction of the loading phase waits for them.
  auto entries = [&](int j) __attribute__((always_inline)) {
    return *(const CONST_AS SVec<4>*)(pl_ent + e0 + 4 * (2 * j + grp));
  };
  auto valid = [&](const SVec<4>& raw, int j) __attribute__((always_inline)) {
    const int es = e0 + 4 * (2 * j + grp);
    SVec<4> r;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) r[pp] = es + pp < e1 ? raw[pp] : 0;
    return r;
  };
  auto mine = [&](const SVec<4>& raw, int j) __attribute__((always_inline)) {
    const int e = e0 + 4 * (2 * j + grp) + wr;
    const int w = wr == 0 ? raw[0] : (wr == 1 ? raw[1] : (wr == 2 ? raw[2] : raw[3]));
    return e < e1 ? w : 0;
  };

  // Loads of this wave's page (entry ent) of a stage: per-lane offsets first (prep), then one
  // 1 KB global->LDS load per call of fire.  Stages past the list have zero entries: every row
  // then loads token 0 (or slot 0), which nobody reads.  The loads are never skipped, so every
  // phase leaves the same number in flight.  A CU accepts such loads at a limited rate and a
  // wave stalls while its load waits, so each phase spreads its loads over its work.
  struct PageLoad {
    uint32_t voff[C::kInst];
    uint32_t soff;
  };
  auto prep = [&](int ent, uint32_t sn_bytes, const uint32_t (&vfull)[C::kInst]) __attribute__((always_inline)) {
    const int nv = ent_nv(ent), slot0 = ent_slot(ent);
    PageLoad L;
    if constexpr (KPERM) {
      // the page's 16 slot tokens as one scalar load (the permutation is padded by 16)
      const SVec<16> tk = *(const CONST_AS SVec<16>*)(kperm + slot0);
#pragma unroll
      for (int n = 0; n < C::kInst; ++n) {
        int tok = tk[n * C::kRowsPerInst];
#pragma unroll
        for (int r = 1; r < C::kRowsPerInst; ++r) tok = ld_lr == r ? tk[n * C::kRowsPerInst + r] : tok;
        tok = ld_rip[n] < nv ? tok : tk[0];
        L.voff[n] = __umul24((uint32_t)tok, sn_bytes) + ld_cb[n];
      }
      L.soff = 0;
    } else {
#pragma unroll
      for (int n = 0; n < C::kInst; ++n) L.voff[n] = ld_rip[n] < nv ? vfull[n] : (uint32_t)ld_cb[n];
      L.soff = (uint32_t)slot0 * sn_bytes;
    }
    return L;
  };
  auto fire = [&](const PageLoad& L, const __amdgpu_buffer_rsrc_t& rsrc, uint8_t* buf, int n) __attribute__((always_inline)) {
    if (n < C::kInst)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)(buf + woff + n * C::kRowsPerInst * C::kRowBytes), 16,
                                               (int)L.voff[n], (int)L.soff, 0, 0);
  };
  auto issue = [&](int ent, const __amdgpu_buffer_rsrc_t& rsrc, uint32_t sn_bytes, const uint32_t (&vfull)[C::kInst],
                   uint8_t* buf) __attribute__((always_inline)) {
    const PageLoad L = prep(ent, sn_bytes, vfull);
#pragma unroll
    for (int n = 0; n < C::kInst; ++n) fire(L, rsrc, buf, n);
  };

  // ---- per-wave state: softmax of the wave's keys, O^T, P of the last stage ----
  float mref = kNegInf;  // reference max, scaled to exp2 units
  float l_run = 0.f;
  f32x16 oacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) oacc[db] = f32x16{};
  f32x16 sacc[JB];  // S^T of the stage; after the vector phase, its P (fp32) until the next P.V
  const float sl2 = p.scale_log2;

  int nbar = 0;
  auto bar = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    ++nbar;
  };

  // Per-lane LDS byte offsets inside the group's stage, so that slot arrays, key blocks and
  // 16-key chunks all become immediate offsets of a few address registers.  K operand of
  // k-step s: row 32 kh + lane % 32 (+ 32 per key block), logical chunk 2s + hh.  V^T operand
  // of d block db: transposed reads of keys 4hh + v_rr and 4hh + v_rr + 8 (+ 16 per chunk).
  // A row's swizzle depends only on its low four bits, which the block and chunk steps keep.
  uint32_t kofs[C::kDS], vofa[C::kDB], vofb[C::kDB];
  {
    const int r = lane & 31;
#pragma unroll
    for (int s = 0; s < C::kDS; ++s)
      kofs[s] = goff + (32 * kh + r) * C::kRowBytes + (((2 * s + hh) ^ swz<D>(r)) * 16);
    const int v_rr = (lane & 15) >> 2, v_qq = lane & 3, v_dsub = (lane >> 4) & 1;
    const int key_a = 4 * hh + v_rr, key_b = key_a + 8;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) {
      const int lc = 4 * db + 2 * v_dsub + (v_qq >> 1);
      const int off_in = (v_qq & 1) * 8;
      vofa[db] = goff + key_a * C::kRowBytes + ((lc ^ swz<D>(key_a)) * 16) + off_in;
      vofb[db] = goff + key_b * C::kRowBytes + ((lc ^ swz<D>(key_b)) * 16) + off_in;
    }
  }

  // V^T operand (16-key chunk c of the wave's keys, d block db), read straight from the V
  // stage with two transposing reads: per-lane offsets with the wave's key half folded in.
  uint32_t vofa_w[C::kDB], vofb_w[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) {
    vofa_w[db] = vofa[db] + (R64 ? 2 * kh * 16 * C::kRowBytes : 0);
    vofb_w[db] = vofb[db] + (R64 ? 2 * kh * 16 * C::kRowBytes : 0);
  }

  // Matrix phase: O^T += V^T P^T over the V stage at vb (PV), then S^T = K Q^T over the K
  // stage at kb (QK).  The products run as one list (PV: 16-key chunk c, d block db; QK:
  // k-step s, key block j) whose operands are read kLead products ahead of their use, so
  // the matrix core does not stall on LDS latency between products.  Without ACT (a wave
  // with no valid rows) the phase issues only the loads.
  constexpr int kNPV = 2 * JB * C::kDB, kNQK = JB * C::kDS, kLead = 2;
  auto mphase = [&](const uint8_t* kb, const uint8_t* vb, auto pv_tag, auto qk_tag, const PageLoad* ldk, uint8_t* kdst,
                    auto act_tag) __attribute__((always_inline)) {
    constexpr bool PV = decltype(pv_tag)::value, QK = decltype(qk_tag)::value, ACT = decltype(act_tag)::value;
    constexpr int n0 = PV ? 0 : kNPV;
    constexpr int n1 = QK ? kNPV + kNQK : kNPV;
    constexpr int kSpread = (n1 - n0) / C::kInst;  // one load before every kSpread-th product
    static_assert(kSpread >= 1, "a product per load");
    if constexpr (!ACT) {
      if (ldk) {
#pragma unroll
        for (int n = 0; n < C::kInst; ++n) fire(*ldk, krsrc, kdst, n);
      }
      return;
    }
    // The SIMD's arbiter favours older waves; raising the matrix wave's priority keeps its
    // MFMAs flowing whichever group is in the vector phase.
    __builtin_amdgcn_s_setprio(2);
    // P of the previous stage (fp32 in sacc) as bf16 operands, and its row sum: vector work
    // that this wave's idle VALU slots absorb while its MFMAs run.  The sum is taken over the
    // fp32 probabilities: with bf16 ones a row of few keys would carry up to 2^-9 relative
    // error into its log-sum-exp.
    bf16x8 pbuf[2 * JB];
    if constexpr (PV) {
#pragma unroll
      for (int kb2 = 0; kb2 < JB; ++kb2)
#pragma unroll
        for (int e = 0; e < 16; ++e) pbuf[2 * kb2 + (e >> 3)][e & 7] = (__bf16)sacc[kb2][e];
      if constexpr (JB == 2)
        l_run += sum16v(sacc[0]) + sum16v(sacc[1]);
      else
        l_run += sum16v(sacc[0]);
    }
    bf16x8 ring[kLead + 1];
    auto load = [&](auto it) __attribute__((always_inline)) {
      constexpr int i = decltype(it)::value;
      if constexpr (i < kNPV) {
        constexpr int c = i / C::kDB, db = i % C::kDB;
        const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(vb + vofa_w[db] + c * 16 * C::kRowBytes));
        const bf16x4 vq = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(vb + vofb_w[db] + c * 16 * C::kRowBytes));
        ring[(i - n0) % (kLead + 1)] = bf16x8{va[0], va[1], va[2], va[3], vq[0], vq[1], vq[2], vq[3]};
      } else {
        constexpr int s = (i - kNPV) / JB, j = (i - kNPV) % JB;
        ring[(i - n0) % (kLead + 1)] = *reinterpret_cast<const bf16x8*>(kb + kofs[s] + j * 32 * C::kRowBytes);
      }
    };
    auto mma = [&](auto it) __attribute__((always_inline)) {
      constexpr int i = decltype(it)::value;
      const bf16x8 a = ring[(i - n0) % (kLead + 1)];
      if constexpr (i < kNPV) {
        constexpr int c = i / C::kDB, db = i % C::kDB;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pbuf[c], oacc[db], 0, 0, 0);
      } else {
        constexpr int s = (i - kNPV) / JB, j = (i - kNPV) % JB;
        sacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], s == 0 ? f32x16{} : sacc[j], 0, 0, 0);
      }
    };
    static_for<n0, (n0 + kLead < n1 ? n0 + kLead : n1)>(load);
    static_for<n0, n1>([&](auto it) __attribute__((always_inline)) {
      constexpr int i = decltype(it)::value;
      if constexpr ((i - n0) % kSpread == 0) {
        constexpr int tt = (i - n0) / kSpread;
        if constexpr (tt < C::kInst) {
          if (ldk) fire(*ldk, krsrc, kdst, tt);
        }
      }
      if constexpr (i + kLead < n1) load(IntTag<i + kLead>{});
      mma(it);
    });
    // keep the order: operand reads kLead products ahead of the MFMAs, loads spread out
    static_for<n0, (n0 + kLead < n1 ? n0 + kLead : n1)>([&](auto it) __attribute__((always_inline)) {
      constexpr int i = decltype(it)::value;
      __builtin_amdgcn_sched_group_barrier(0x100, i < kNPV ? 2 : 1, 0);
    });
    static_for<n0, n1>([&](auto it) __attribute__((always_inline)) {
      constexpr int i = decltype(it)::value;
      if constexpr ((i - n0) % kSpread == 0 && (i - n0) / kSpread < C::kInst) {
        if (ldk) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      if constexpr (i + kLead < n1) __builtin_amdgcn_sched_group_barrier(0x100, i + kLead < kNPV ? 2 : 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    });
    // the products stay in this phase (see pin_vector_phase)
#pragma unroll
    for (int j = 0; j < JB; ++j) pin(sacc[j]);
    pin(l_run);
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) pin(oacc[db]);
    __builtin_amdgcn_s_setprio(0);
  };

  // Phases only overlap if each one's instructions stay in it.  The compiler would otherwise
  // sink the exponentials and conversions of a vector phase down to their use by the next
  // matrix phase's MFMAs (and could hoist matrix work the other way), so the results of each
  // phase are tied to its end by empty asm statements that use them.
  auto pin_vector_phase = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < JB; ++j) pin(sacc[j]);
    pin(l_run);
    pin(mref);
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) pin(oacc[db]);
  };

  // Mask, online softmax and P (in place, fp32) of a stage with page entries ev (S^T in sacc);
  // its row sum and bf16 conversion happen in the next matrix phase.
  auto softmax = [&](const SVec<4>& raw, int j) __attribute__((always_inline)) {
    // the planner flags stages with a partial page or a cut-short end (bit 31 of the first
    // entry); causal problems also mask stages whose keys may follow a query
    bool need = raw[0] < 0;
    if (p.causal) {
      const SVec<4> ev = valid(raw, j);
      int maxkey = -1;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int nv = ent_nv(ev[pp]);
        const int last = ent_slot(ev[pp]) + nv - 1;
        maxkey = (nv > 0 && last > maxkey) ? last : maxkey;
      }
      need |= p.qperm ? true : ((int64_t)maxkey > minq_pos);
    }
    if (need) {
      const SVec<4> ev = valid(raw, j);
      // entries of this wave's pages: 2 (kb + kh) and 2 (kb + kh) + 1 for key block kb
      int ment[2 * JB];
      if constexpr (R64) {
        ment[0] = kh ? ev[2] : ev[0];
        ment[1] = kh ? ev[3] : ev[1];
      } else {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) ment[pp] = ev[pp];
      }
#pragma unroll
      for (int kb2 = 0; kb2 < JB; ++kb2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // key 32kb + 8i + 4hh + jj is row 8(i&1) + 4hh + jj of page 2kb + i/2
          const int ent = ment[2 * kb2 + (i >> 1)];
          int lim = (ent & 31) - 1;
          if (p.causal) lim = min(lim, thr - ent_slot(ent));
          const int rip0 = 8 * (i & 1) + 4 * hh;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (rip0 + jj > lim) sacc[kb2][4 * i + jj] = kNegInf;
        }
      }
    }
    float mt = max16(sacc[0]);
    if constexpr (JB == 2) mt = fmaxf(mt, max16(sacc[1]));
    mt = xor32_max(mt) * sl2;
    const bool grow = mt > mref + kLazySlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(mref - mt) : 1.f;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) oacc[db] *= alpha;
      l_run *= alpha;
      mref = grow ? mt : mref;
    }
    const float nb = mref == kNegInf ? 0.f : -mref;
    // all scalings, then all exponentials, each in place: 32 independent operations per step
    // instead of 32 dependent pairs through one temporary register
#pragma unroll
    for (int kb2 = 0; kb2 < JB; ++kb2)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb2][e] = __builtin_fmaf(sacc[kb2][e], sl2, nb);
#pragma unroll
    for (int j2 = 0; j2 < JB; ++j2) pin(sacc[j2]);
#pragma unroll
    for (int kb2 = 0; kb2 < JB; ++kb2)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb2][e] = __builtin_amdgcn_exp2f(sacc[kb2][e]);
    pin_vector_phase();
  };

  // Load schedule of local stage j: matrix phase j issues K(j + 1), spread over its products
  // (its slot held K(j - 1), read in matrix phase j - 1); vector phase j issues V(j + 1) at
  // its start (its slot held V(j - 1), read by the P.V products of matrix phase j, which the
  // barrier between the two phases has closed).  Vector phase j ends by waiting for K(j + 1),
  // and with it for V(j), issued before it.  Page entries of stage j + 3 are loaded in vector
  // phase j, where no LDS wait can cover the scalar load.
  if (ns > 0) {
    SVec<4> x0 = entries(0), x1 = entries(1), x2 = entries(2);  // raw entries of stages j, j + 1, j + 2
    issue(mine(x0, 0), krsrc, p.k_sn_bytes, ld_vk, sk0);
    issue(mine(x0, 0), vrsrc, p.v_sn_bytes, ld_vv, sv0);
    wait_vmcnt<C::kInst>();  // K of stage 0 landed
    bar();
    if (grp == 1) bar();  // group 1 runs one phase behind
    // the walk; a wave whose row group holds only padding runs it without products
    auto walk = [&](auto act_tag) __attribute__((always_inline)) {
      constexpr bool ACT = decltype(act_tag)::value;
      // matrix phase: P.V of the previous stage (if PV), S of the stage in kbuf (if QK), loads
      // of stage jn (entry word ent) into kdst / vdst
      auto mph = [&](auto pv_tag, auto qk_tag, const uint8_t* kbuf, const uint8_t* vbuf, int ent, uint8_t* kdst)
                     __attribute__((always_inline)) {
        const PageLoad lk = prep(ent, p.k_sn_bytes, ld_vk);
        mphase(kbuf, vbuf, pv_tag, qk_tag, &lk, kdst, act_tag);
        bar();
      };
      // vector phase of stage j: V of stage j + 1 (entry word ent) loaded into vdst, entries of
      // stage j + 3 loaded, softmax with raw entries ej
      auto vph = [&](int j, const SVec<4>& ej, int ent, uint8_t* vdst) __attribute__((always_inline)) {
        issue(ent, vrsrc, p.v_sn_bytes, ld_vv, vdst);
        __builtin_amdgcn_sched_barrier(0);
        const SVec<4> next = entries(j + 3);
        if constexpr (ACT) softmax(ej, j);
        wait_vmcnt<C::kInst>();  // K of the next stage landed (V of this one was issued before it)
        bar();
        return next;
      };
      mph(BoolTag<false>{}, BoolTag<true>{}, sk0, sv0, mine(x1, 1), sk1);
      const SVec<4> x3 = vph(0, x0, mine(x1, 1), sv1);
      x0 = x1;
      x1 = x2;
      x2 = x3;
      int j = 1;
      for (; j + 1 < my_n; j += 2) {
        mph(BoolTag<true>{}, BoolTag<true>{}, sk1, sv0, mine(x1, j + 1), sk0);  // P.V of j - 1, S of j (odd)
        const SVec<4> x3n = vph(j, x0, mine(x1, j + 1), sv0);
        mph(BoolTag<true>{}, BoolTag<true>{}, sk0, sv1, mine(x2, j + 2), sk1);  // P.V of j, S of j + 1 (even)
        const SVec<4> x4 = vph(j + 1, x1, mine(x2, j + 2), sv1);
        x0 = x2;
        x1 = x3n;
        x2 = x4;
      }
      if (j < my_n) {
        mph(BoolTag<true>{}, BoolTag<true>{}, sk1, sv0, mine(x1, j + 1), sk0);
        vph(j, x0, mine(x1, j + 1), sv0);
      }
      // P.V of the last stage, my_n - 1, whose V is in slot (my_n - 1) & 1
      if (my_n & 1)
        mphase(sk0, sv0, BoolTag<true>{}, BoolTag<false>{}, nullptr, nullptr, act_tag);
      else
        mphase(sk0, sv1, BoolTag<true>{}, BoolTag<false>{}, nullptr, nullptr, act_tag);
      bar();
    };
    if (my_n > 0) {
      if (active)
        walk(BoolTag<true>{});
      else
        walk(BoolTag<false>{});
    }
    // both groups pass the same number of barriers
    const int n0 = (ns + 1) >> 1, n1 = ns >> 1;
    const int c0 = 2 * n0 + 2, c1 = n1 > 0 ? 2 * n1 + 3 : 2;
    const int total = c0 > c1 ? c0 : c1;
    while (nbar < total) bar();
    wait_vmcnt<0>();  // loads past the list may still be landing in the stage buffers
  }

  // ---- finish: combine lane halves, merge the states of each row group, write O and LSE ----
  // States: one per group (128-row tiles), one per (group, key half) (64-row tiles).  Every
  // state but (group 0, key half 0) goes to LDS as a record -- O^T in one of the four stage
  // arrays, max and sum in the record array -- and that wave combines them.
  float l_tot = xor32_sum(l_run);
  constexpr int kStates = R64 ? 4 : 2;                 // states per row group
  const int sidx = R64 ? (2 * grp + kh) : grp;         // this wave's state
  __syncthreads();
  if (sidx != 0) {
    const int rec = rg * (kStates - 1) + sidx - 1;     // 0 .. 3 (128-row) or 0 .. 5 (64-row)
    uint8_t* arr = (rec >> 1) == 0 ? sk0 : ((rec >> 1) == 1 ? sk1 : ((rec >> 1) == 2 ? sv0 : sv1));
    float* ob = reinterpret_cast<float*>(arr + (rec & 1) * C::kRecord);
    float* mlb = reinterpret_cast<float*>(sml) + rec * 128;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) ob[(db * 16 + e) * 64 + lane] = oacc[db][e];
    mlb[lane] = mref;
    mlb[64 + lane] = l_tot;
  }
  __syncthreads();
  if (sidx != 0) return;
  float mm = mref;
#pragma unroll
  for (int s = 1; s < kStates; ++s) mm = fmaxf(mm, reinterpret_cast<const float*>(sml)[(rg * (kStates - 1) + s - 1) * 128 + lane]);
  const float mu = (mm == kNegInf) ? 0.f : mm;
  {
    const float a0 = __builtin_amdgcn_exp2f(mref - mu);
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) oacc[db] *= a0;
    l_tot *= a0;
  }
#pragma unroll
  for (int s = 1; s < kStates; ++s) {
    const int rec = rg * (kStates - 1) + s - 1;
    const uint8_t* arr = (rec >> 1) == 0 ? sk0 : ((rec >> 1) == 1 ? sk1 : ((rec >> 1) == 2 ? sv0 : sv1));
    const float* ob = reinterpret_cast<const float*>(arr + (rec & 1) * C::kRecord);
    const float* mlb = reinterpret_cast<const float*>(sml) + rec * 128;
    const float a1 = __builtin_amdgcn_exp2f(mlb[lane] - mu);
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] += ob[(db * 16 + e) * 64 + lane] * a1;
    l_tot += mlb[64 + lane] * a1;
  }

  if (!qvalid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  __bf16* op = reinterpret_cast<__bf16*>(p.o) + (int64_t)b * p.o_sb + (int64_t)qtok * p.o_sn + (int64_t)h * p.o_sh;
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 v4;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) v4[jj] = (__bf16)(oacc[db][4 * i + jj] * inv);
      *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * i + 4 * hh) = v4;
    }
  }
  if (hh == 0) {
    const float lse = l_tot > 0.f ? mm * kLn2 + __logf(l_tot) : kNegInf;
    p.lse[((int64_t)b * p.Hq + h) * p.Nq + qtok] = lse;
  }
}

// Block blk runs on XCD blk % 8 and is that XCD's (blk / 8)-th block.  The XCDs are split
// into groups of kXcdShare; the groups take the (batch, head) slices in turn (group g: slices
// g, g + 8 / kXcdShare, ...), and inside a group XCD x takes a contiguous chunk of each
// slice's Q tiles.  Consecutive tiles of one XCD -- neighbouring Q blocks, whose K/V windows
// overlap -- share its L2, and the slices in flight at a time, whose K/V the L2 misses
// fetch, are few: 8 / kXcdShare of them.
struct XcdList {
  int c0, len;  // this XCD's tiles of each slice: [c0, c0 + len)
  int g, G;     // its group, and the number of groups
  int count;    // items of this XCD: len x slices of the group
};
__host__ __device__ inline XcdList xcd_list(int x, int n_qtiles, int BH) {
  constexpr int S = kXcdShare;
  XcdList l;
  const int px = x % S;
  l.G = 8 / S;
  l.g = x / S;
  l.c0 = px * n_qtiles / S;
  l.len = (px + 1) * n_qtiles / S - l.c0;
  const int nh = BH > l.g ? (BH - l.g + l.G - 1) / l.G : 0;
  l.count = l.len * nh;
  return l;
}
// work index (slice * n_qtiles + tile) of item i < l.count of an XCD's list
__device__ __forceinline__ int xcd_work(const XcdList& l, int i, int n_qtiles) {
  const int j = i / l.len;
  return (l.g + j * l.G) * n_qtiles + l.c0 + (i - j * l.len);
}
// blocks per XCD a launch needs: the longest XCD list (of one or two shapes)
static int xcd_rounds(int n1, int n2, int BH) {
  int m = 0;
  for (int x = 0; x < 8; ++x) m = std::max(m, xcd_list(x, n1, BH).count + xcd_list(x, n2, BH).count);
  return m;
}

// Tiles of one shape (R64: the 64-row tiles), one workgroup per tile.
template <int D, bool KPERM, bool R64>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) fwd_kernel_pp(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sk0[2 * PPCfg<D>::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sk1[2 * PPCfg<D>::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sv0[2 * PPCfg<D>::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sv1[2 * PPCfg<D>::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sml[PPCfg<D>::kMlBytes];
  const PPSmem<D> sm{sk0, sk1, sv0, sv1, sml};
  const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
  const XcdList l = xcd_list(x, p.n_qtiles, p.B * p.Hq);
  if (i >= l.count) return;  // the grid covers the longest XCD list
  pp_walk<D, KPERM, R64>(p, (const CONST_AS int32_t*)p.qtiles, p.n_qtiles, xcd_work(l, i, p.n_qtiles), sm);
}

// Both shapes in one launch: the 128-row tiles (qtiles, n_qtiles per slice) and the 64-row
// tiles (qtiles2, n_qtiles2).  Each XCD takes its share of each kind, its 128-row tiles
// first: the shorter 64-row tiles then fill the end of the launch, where XCDs would
// otherwise wait for each other's last tiles.
template <int D, bool KPERM>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) fwd_kernel_pp_fused(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sk0[2 * PPCfg<D>::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sk1[2 * PPCfg<D>::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sv0[2 * PPCfg<D>::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sv1[2 * PPCfg<D>::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sml[PPCfg<D>::kMlBytes];
  const PPSmem<D> sm{sk0, sk1, sv0, sv1, sml};
  const int x = blockIdx.x & 7, i = blockIdx.x >> 3, BH = p.B * p.Hq;
  const XcdList a = xcd_list(x, p.n_qtiles, BH);
  if (i < a.count) {
    pp_walk<D, KPERM, false>(p, (const CONST_AS int32_t*)p.qtiles, p.n_qtiles, xcd_work(a, i, p.n_qtiles), sm);
    return;
  }
  const XcdList c = xcd_list(x, p.n_qtiles2, BH);
  if (i - a.count < c.count)
    pp_walk<D, KPERM, true>(p, (const CONST_AS int32_t*)p.qtiles2, p.n_qtiles2, xcd_work(c, i - a.count, p.n_qtiles2), sm);
}

template <int D, int NRG, int NKG, int KB>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  if (p.n_work <= 0) return hipSuccess;
  if (p.kperm)
    hipLaunchKernelGGL((fwd_kernel<D, NRG, NKG, KB, true>), dim3(p.n_work), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_kernel<D, NRG, NKG, KB, false>), dim3(p.n_work), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool R64>
static hipError_t launch_pp(const FwdParams& p, hipStream_t stream) {
  if (p.n_work <= 0) return hipSuccess;
  const dim3 grid(8 * xcd_rounds(p.n_qtiles, 0, p.B * p.Hq));
  if (p.kperm)
    hipLaunchKernelGGL((fwd_kernel_pp<D, true, R64>), grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_kernel_pp<D, false, R64>), grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_pp_fused(const FwdParams& p, hipStream_t stream) {
  if (p.n_work + p.n_work2 <= 0) return hipSuccess;
  const dim3 grid(8 * xcd_rounds(p.n_qtiles, p.n_qtiles2, p.B * p.Hq));
  if (p.kperm)
    hipLaunchKernelGGL((fwd_kernel_pp_fused<D, true>), grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_kernel_pp_fused<D, false>), grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

// The ping-pong walk runs both shapes unless keys are permuted under a causal mask (its mask
// reads no key tokens) or the permuted offsets would not fit 24-bit products; those problems
// go to the 4-wave kernel above (128-row tiles: 4 row groups x 128-key tiles; 64-row tiles:
// 2 row groups x 2 key groups of 64 keys).
static bool pp_supported(const FwdParams& p) {
  if (!p.kperm) return true;
  return !p.causal && p.Nk < (1 << 24) && p.k_sn_bytes < (1u << 24) && p.v_sn_bytes < (1u << 24);
}

template <int D>
static hipError_t launch_shape_d(const FwdParams& p, int shape, hipStream_t stream) {
  if (shape == 0) return pp_supported(p) ? launch_pp<D, false>(p, stream) : launch_one<D, 4, 1, 4>(p, stream);
  return pp_supported(p) ? launch_pp<D, true>(p, stream) : launch_one<D, 2, 2, 2>(p, stream);
}

hipError_t launch_fwd_shape(const FwdParams& p, int shape, int d, hipStream_t stream) {
  return d == 128 ? launch_shape_d<128>(p, shape, stream) : launch_shape_d<64>(p, shape, stream);
}

// Both shapes: one fused launch when the ping-pong walk supports the problem, else one
// launch per shape.  p describes the 128-row tiles (qtiles, n_qtiles, n_work) and p.qtiles2,
// n_qtiles2, n_work2 the 64-row ones.
hipError_t launch_fwd(const FwdParams& p, int d, hipStream_t stream) {
  if (pp_supported(p)) return d == 128 ? launch_pp_fused<128>(p, stream) : launch_pp_fused<64>(p, stream);
  FwdParams p2 = p;
  p2.qtiles = p.qtiles2;
  p2.n_qtiles = p.n_qtiles2;
  p2.n_work = p.n_work2;
  hipError_t e = launch_fwd_shape(p, 0, d, stream);
  if (e != hipSuccess) return e;
  return launch_fwd_shape(p2, 1, d, stream);
}

}  // namespace bsattn
