// Exact block-sparse attention forward for gfx950 (MI355X).
//
// One workgroup (4 waves) owns one Q tile of one (batch, head) and walks its K tiles.
// A K tile is 8 or 16 page-list entries; each entry is a 16-row K/V page of one block,
// so a tile packs pages of several logical blocks (KPage abstract, zhuanzhiai page 1,
// sentence 2).  Pages are gathered from HBM straight into LDS (global_load_lds, 16 bytes
// per lane): nothing compacted is ever written back.  Q tiles come in two shapes
// (sentence 3): 128 rows x 128 keys (4 row groups of 32 queries, one per wave) and 64 rows
// x 256 keys (2 row groups x 2 key groups; the key groups keep separate softmax states
// that are merged at the end).  Exact masking (sentence 4) clears empty page slots and,
// for causal problems, keys after the query.
//
// Per wave and K tile the work is 32 queries x 128 keys:
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

#include <cstdint>

#include "kernel_params.hpp"

namespace bsattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
// N consecutive dwords with dword alignment: one scalar load (s_load_dwordxN) when uniform
template <int N>
using SVec = int __attribute__((ext_vector_type(N), aligned(4)));

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))
#define CONST_AS __attribute__((address_space(4)))

constexpr float kNegInf = -__builtin_huge_valf();

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS hand-off: publish this wave's LDS writes, then s_barrier.
// Global->LDS loads are waited for explicitly (wait_vmcnt) before calling it.  The empty
// asm statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt/expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// XOR swizzle of the 16-byte chunk index inside an LDS row (d = 128: 16 chunks, d = 64:
// 8 chunks).  Sixteen consecutive rows read at one logical chunk hit sixteen distinct
// chunk slots (the K operand reads), and the 8 rows x 4 chunks of one transposed V read
// land on every slot of a 256-byte bank line twice.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    const int m = (row >> 1) & 7;
    return ((m & 1) << 2) | ((m >> 1) & 3);
  }
}

// Lane l gets max / sum of its value and lane (l ^ 32)'s (v_permlane32_swap).
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max / sum of 16 accumulator values as shallow trees (short dependency chains).
__device__ __forceinline__ float max16(const f32x16& v) {
  const float a = fmaxf(fmaxf(v[0], v[1]), v[2]), b2 = fmaxf(fmaxf(v[3], v[4]), v[5]);
  const float c = fmaxf(fmaxf(v[6], v[7]), v[8]), d = fmaxf(fmaxf(v[9], v[10]), v[11]);
  const float e = fmaxf(fmaxf(v[12], v[13]), v[14]);
  return fmaxf(fmaxf(fmaxf(a, b2), c), fmaxf(fmaxf(d, e), v[15]));
}
__device__ __forceinline__ float sum16(const float* x) {
  const float a = (x[0] + x[1]) + (x[2] + x[3]), b2 = (x[4] + x[5]) + (x[6] + x[7]);
  const float c = (x[8] + x[9]) + (x[10] + x[11]), d = (x[12] + x[13]) + (x[14] + x[15]);
  return (a + b2) + (c + d);
}

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
  // two workgroups per CU when the LDS allows it
  // workgroups per CU that the LDS allows (at most 3: the register budget of 168)
  static constexpr int kLds = 2 * kBufBytes + kTileK * 4;
#ifdef BSATTN_WPE_MAX
  static constexpr int kWpeMax = BSATTN_WPE_MAX;
#else
  static constexpr int kWpeMax = 2;  // three waves per SIMD would leave 168 VGPRs: too few
#endif
  static constexpr int kWavesPerEU =
      (kWpeMax >= 3 && 3 * kLds <= 160 * 1024) ? 3 : ((kWpeMax >= 2 && 2 * kLds <= 160 * 1024) ? 2 : 1);
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
        const int tok = p.kperm[(ent >> 5) + (rip < nv ? rip : 0)];
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
      const int last = (ment[pp] >> 5) + nv - 1;
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
  // data that the mask removes.
  auto issue = [&](const __amdgpu_buffer_rsrc_t& rsrc, uint32_t sn_bytes, const uint32_t (&vfull)[kPeriod],
                   uint8_t* buf) {
    if (KPERM || !ents_full) {
#pragma unroll
      for (int n = 0; n < C::kInst; ++n) {
        uint32_t voff, soff;
        if constexpr (KPERM) {
          voff = (uint32_t)ldtok[n] * sn_bytes + ld_cb[n % kPeriod];
          soff = 0;
        } else {
          const int ent = ents[(n * C::kRowsPerInst) >> 4];
          voff = ld_rip[n % kPeriod] < (ent & 31) ? vfull[n % kPeriod] : (uint32_t)ld_cb[n % kPeriod];
          soff = (uint32_t)(ent >> 5) * sn_bytes;
        }
        uint8_t* dst = buf + (wave * C::kRowsPerWave + n * C::kRowsPerInst) * C::kRowBytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)dst, 16, (int)voff, (int)soff, 0, 0);
      }
    } else {
#pragma unroll
      for (int n = 0; n < C::kInst; ++n) {
        const uint32_t soff = (uint32_t)(ents[(n * C::kRowsPerInst) >> 4] >> 5) * sn_bytes;
        uint8_t* dst = buf + (wave * C::kRowsPerWave + n * C::kRowsPerInst) * C::kRowBytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)dst, 16, (int)vfull[n % kPeriod], (int)soff, 0, 0);
      }
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

  for (int kt = 0; kt < nkt; ++kt) {
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
            if (p.causal) lim = min(lim, thr - (ent >> 5));
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
    if (kt + 1 < nkt) {
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

    lds_barrier();  // every wave is done with the V buffer
    if (kt + 1 < nkt) issue(vrsrc, p.v_sn_bytes, ld_vv, smem_v);
  }

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

template <int D, int NRG, int NKG, int KB>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  if (p.n_work <= 0) return hipSuccess;
  if (p.kperm)
    hipLaunchKernelGGL((fwd_kernel<D, NRG, NKG, KB, true>), dim3(p.n_work), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_kernel<D, NRG, NKG, KB, false>), dim3(p.n_work), dim3(256), 0, stream, p);
  return hipGetLastError();
}

#ifndef BSATTN_KB128
#define BSATTN_KB128 4
#endif
#ifndef BSATTN_KB64
#define BSATTN_KB64 2
#endif

hipError_t launch_fwd_shape(const FwdParams& p, int shape, int d, hipStream_t stream) {
  if (d == 128)
    return shape == 0 ? launch_one<128, 4, 1, BSATTN_KB128>(p, stream) : launch_one<128, 2, 2, BSATTN_KB64>(p, stream);
  return shape == 0 ? launch_one<64, 4, 1, BSATTN_KB128>(p, stream) : launch_one<64, 2, 2, BSATTN_KB64>(p, stream);
}

}  // namespace bsattn
