// Exact block-sparse attention for decode and other small query blocks, gfx950 (MI355X).
//
// With a handful of queries per Q block the forward's 64- or 128-row tiles are almost empty
// and every query head of a KV group would read the same selected pages again.  Here the
// query heads of one KV group that share a selection (one indexing query per KV group,
// CISA abstract, fugumt page 4, sentences 4-5) are stacked into the 32 columns of one tile:
// column c = (head h0 + c / n, query c % n) of a Q block with n rows, n * (Hq / Hkv) <= 32.
// The pages of the block's list are read once for all of them.  The regime is bound by HBM
// (8 FLOP per K/V byte for 8 stacked heads), so the list is split over many workgroups:
//   fwd_decode_kernel  one workgroup (4 waves) per (batch, KV group, Q block, split); each
//                      wave walks 32 keys (2 pages) of every 128-key stage of its split with
//                      its own online softmax -- S^T = K Q^T and O^T += V^T P^T on
//                      v_mfma_f32_32x32x16_bf16 as in the forward -- and the four states are
//                      merged in LDS into one partial (max, sum, unnormalised O) per split.
//   decode_merge_kernel  combines the splits of a (batch, group, block) exactly:
//                      M = max m_s, O = sum 2^(m_s - M) O_s / sum 2^(m_s - M) l_s.
// Pages go through registers into a wave-private LDS region, so the walk needs no
// workgroup barrier and never waits for loads behind an LDS read.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "device_common.hpp"
#include "kernel_params.hpp"

namespace bsattn {

typedef unsigned int u32x4d __attribute__((ext_vector_type(4)));

template <int D>
struct DecCfg {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;
  static constexpr int kRowsPerInst = 64 / kChunks;
  static constexpr int kInst = 32 / kRowsPerInst;  // loads per tensor for a wave's 32 keys
  static constexpr int kWaveBuf = 32 * kRowBytes;
  static constexpr int kDS = D / 16;
  static constexpr int kDB = D / 32;
  static constexpr int kSlots = kDB * 16 + 2;  // merge record per wave and lane: O^T, max, sum
  static constexpr int kPages = 8 * kWaveBuf;  // K and V regions of the four waves
  static constexpr int kMerge = 4 * kSlots * 64 * 4;
  static constexpr int kLds = kPages > kMerge ? kPages : kMerge;
};

// two waves per SIMD (two workgroups per CU): twice the loads in flight in this HBM-bound walk
template <int D, bool KPERM>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) fwd_decode_kernel(DecodeParams p) {
  using C = DecCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLds];
  uint8_t* sk = smem;
  uint8_t* sv = smem + 4 * C::kWaveBuf;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5;
  const CONST_AS int32_t* pl_ent = (const CONST_AS int32_t*)p.pl_ent;
  const CONST_AS int32_t* pl_ptr = (const CONST_AS int32_t*)p.pl_ptr;
  const CONST_AS int32_t* qtiles = (const CONST_AS int32_t*)p.qtiles;

  const int work = blockIdx.x;  // ((b * Hkv + g) * n_qtiles + t) * n_splits + split
  const int split = work % p.n_splits;
  const int rest = work / p.n_splits;
  const int t = rest % p.n_qtiles;
  const int bg = rest / p.n_qtiles;
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int row0 = qtiles[4 * t], n = qtiles[4 * t + 1], qblock = qtiles[4 * t + 2];
  const int unit = (b * p.ub_mul) * p.sel_nh + (g * p.grp) / p.uh_div;
  const int lrow = unit * p.nqb + qblock;
  const int e0 = pl_ptr[lrow], e1 = pl_ptr[lrow + 1];
  const int pb0 = e0 + split * p.pps;
  const int pb1 = min(e1, pb0 + p.pps);
  const int nst = pb1 > pb0 ? (pb1 - pb0 + 7) >> 3 : 0;  // 128-key stages of the split

  // this lane's column: head h0 + c / n, query row c % n of the block
  const int c = lane & 31;
  const bool cvalid = c < p.grp * n;
  const int hi = cvalid ? c / n : 0, qi = cvalid ? c - (c / n) * n : 0;
  const int h = g * p.grp + hi;
  const int qslot = row0 + qi;
  const int qtok = p.qperm ? p.qperm[qslot] : qslot;
  bf16x8 qreg[C::kDS];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb + (int64_t)qtok * p.q_sn +
                       (int64_t)h * p.q_sh + hh * 8;
#pragma unroll
    for (int s = 0; s < C::kDS; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }
  int thr = 0x7ffffffe;
  if (p.causal) {
    const int64_t qpos = p.q_pos0 + (int64_t)qtok;
    thr = qpos < -1 ? -1 : (qpos > 0x7ffffffe ? 0x7ffffffe : (int)qpos);
  }

  // loads: instruction n covers rows n * kRowsPerInst + lr of the wave's 32 keys (page row / 16)
  const int lr = lane / C::kChunks, pc = lane % C::kChunks;
  const char* kslice = reinterpret_cast<const char*>(p.k) + ((int64_t)b * p.k_sb + (int64_t)g * p.k_sh) * 2;
  const char* vslice = reinterpret_cast<const char*>(p.v) + ((int64_t)b * p.v_sb + (int64_t)g * p.v_sh) * 2;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)kslice, (short)0, p.k_extent, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)vslice, (short)0, p.v_extent, 0x00020000);
  u32x4d rk[C::kInst], rv[C::kInst];
  int ent[2];  // page entries of the wave's two pages in the loaded stage
  auto load = [&](int st) {
    const int e = pb0 + 8 * st + 2 * wave;
    ent[0] = e < pb1 ? pl_ent[e] : 0;
    ent[1] = e + 1 < pb1 ? pl_ent[e + 1] : 0;
#pragma unroll
    for (int i = 0; i < C::kInst; ++i) {
      const int row = i * C::kRowsPerInst + lr;
      const int en = (row >> 4) ? ent[1] : ent[0];
      const int rip = row & 15;
      const int slot = ent_slot(en) + (rip < ent_nv(en) ? rip : 0);
      const uint32_t tok = (uint32_t)(KPERM ? p.kperm[slot] : slot);
      const uint32_t cb = (uint32_t)((pc ^ swz<D>(rip)) * 16);
      rk[i] = __builtin_amdgcn_raw_buffer_load_b128(krsrc, (int)(tok * p.k_sn_bytes + cb), 0, 0);
      rv[i] = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, (int)(tok * p.v_sn_bytes + cb), 0, 0);
    }
  };
  uint8_t* mk = sk + wave * C::kWaveBuf;
  uint8_t* mv = sv + wave * C::kWaveBuf;
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < C::kInst; ++i) {
      *reinterpret_cast<u32x4d*>(mk + i * C::kRowsPerInst * C::kRowBytes + lane * 16) = rk[i];
      *reinterpret_cast<u32x4d*>(mv + i * C::kRowsPerInst * C::kRowBytes + lane * 16) = rv[i];
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) oacc[db] = f32x16{};
  const float sl2 = p.scale_log2;
  const int v_rr = (lane & 15) >> 2, v_qq = lane & 3, v_dsub = (lane >> 4) & 1;

  if (nst > 0) load(0);
  for (int st = 0; st < nst; ++st) {
    const int ea = ent[0], eb = ent[1];  // entries of this stage's pages (for the mask)
    store();
    if (st + 1 < nst) load(st + 1);
    // S^T = K Q^T over the wave's 32 keys
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < C::kDS; ++s) {
      const int r = lane & 31;
      const int cc = (2 * s + hh) ^ swz<D>(r);
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(mk + r * C::kRowBytes + cc * 16);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc, 0, 0, 0);
    }
    // register i holds key 8 (i / 4) + 4 hh + i % 4: page i / 8, row key % 16
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int en = (i >> 3) ? eb : ea;
      const int rip = 8 * ((i >> 2) & 1) + 4 * hh + (i & 3);
      bool keep = rip < ent_nv(en);
      if (p.causal) {
        const int slot = ent_slot(en) + rip;
        const int ktok = KPERM ? p.kperm[keep ? slot : 0] : slot;
        keep = keep && ktok <= thr;
      }
      if (!keep) sacc[i] = kNegInf;
    }
    // online softmax of the lane's column (its 16 keys and the other half's 16)
    const float mt = xor32_max(max16(sacc));
    const float m_new = fmaxf(m_run, mt * sl2);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) oacc[db] *= alpha;
    bf16x8 pb[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], sl2, -m_use));
#pragma unroll
    for (int e = 0; e < 16; ++e) pb[e >> 3][e & 7] = (__bf16)sacc[e];
    {
      float tmp[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) tmp[e] = sacc[e];
      l_run += sum16(tmp);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int ka = 16 * half + 4 * hh + v_rr, kb2 = ka + 8;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) {
        const int lc = 4 * db + 2 * v_dsub + (v_qq >> 1);
        const int off_in = (v_qq & 1) * 8;
        LDS_AS bf16x4* pa = (LDS_AS bf16x4*)(mv + ka * C::kRowBytes + ((lc ^ swz<D>(ka)) * 16) + off_in);
        LDS_AS bf16x4* pv = (LDS_AS bf16x4*)(mv + kb2 * C::kRowBytes + ((lc ^ swz<D>(kb2)) * 16) + off_in);
        const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(pa);
        const bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(pv);
        const bf16x8 av = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[half], oacc[db], 0, 0, 0);
      }
    }
  }

  // merge the four waves' states (both lane halves hold halves of the column's sum)
  l_run = xor32_sum(l_run);
  __syncthreads();  // every wave is done with its LDS region
  float* mb = reinterpret_cast<float*>(smem);  // [4 waves][kSlots][64 lanes]
  constexpr int kSlots = C::kSlots;
#pragma unroll
  for (int db = 0; db < C::kDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) mb[(wave * kSlots + db * 16 + e) * 64 + lane] = oacc[db][e];
  mb[(wave * kSlots + C::kDB * 16) * 64 + lane] = m_run;
  mb[(wave * kSlots + C::kDB * 16 + 1) * 64 + lane] = l_run;
  __syncthreads();
  if (wave != 0) return;
  float mw[4], m_all = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = mb[(w * kSlots + C::kDB * 16) * 64 + lane];
    m_all = fmaxf(m_all, mw[w]);
  }
  const float mu = m_all == kNegInf ? 0.f : m_all;
  float aw[4], l_all = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    aw[w] = __builtin_amdgcn_exp2f(mw[w] - mu);
    l_all += aw[w] * mb[(w * kSlots + C::kDB * 16 + 1) * 64 + lane];
  }
  float* op = p.opart + ((int64_t)work * 32 + c) * D;
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 v4;
      float* vv = reinterpret_cast<float*>(&v4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 4 * i + j;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) acc += aw[w] * mb[(w * kSlots + db * 16 + e) * 64 + lane];
        vv[j] = acc;
      }
      *reinterpret_cast<float4*>(op + 32 * db + 8 * i + 4 * hh) = v4;
    }
  }
  if (hh == 0) {
    p.mlpart[((int64_t)work * 32 + c) * 2] = m_all;
    p.mlpart[((int64_t)work * 32 + c) * 2 + 1] = l_all;
  }
}

// one workgroup (4 waves) per (batch, KV group, Q block, 4 stacked columns): a wave per
// column, each lane D / 64 of its values
template <int D>
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeParams p) {
  constexpr int kPer = D / 64;
  const int item = blockIdx.x >> 3;  // (b * Hkv + g) * n_qtiles + t
  const int c = (blockIdx.x & 7) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t = item % p.n_qtiles;
  const int bg = item / p.n_qtiles;
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  const CONST_AS int32_t* qtiles = (const CONST_AS int32_t*)p.qtiles;
  const int row0 = qtiles[4 * t], n = qtiles[4 * t + 1];
  if (c >= p.grp * n) return;  // whole waves
  const int hi = c / n, qi = c - (c / n) * n;
  const int h = g * p.grp + hi;
  const int qslot = row0 + qi;
  const int qtok = p.qperm ? p.qperm[qslot] : qslot;
  const int64_t w0 = (int64_t)item * p.n_splits;
  // split weights 2^(m_s - M): lanes over splits, wave reductions (n_splits <= 256)
  __shared__ float sa[4][256];
  float* wa = sa[threadIdx.x >> 6];
  float M = kNegInf;
  for (int s = lane; s < p.n_splits; s += 64) M = fmaxf(M, p.mlpart[((w0 + s) * 32 + c) * 2]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  const float mu = M == kNegInf ? 0.f : M;
  float L = 0.f;
  for (int s = lane; s < p.n_splits; s += 64) {
    const float a = __builtin_amdgcn_exp2f(p.mlpart[((w0 + s) * 32 + c) * 2] - mu);
    wa[s] = a;
    L += a * p.mlpart[((w0 + s) * 32 + c) * 2 + 1];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) L += __shfl_xor(L, m, 64);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS writes are visible to its own reads
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
#pragma unroll 8
  for (int s = 0; s < p.n_splits; ++s) {
    const float* op = p.opart + ((w0 + s) * 32 + c) * D + lane * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[e] += wa[s] * op[e];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  __bf16* dst = reinterpret_cast<__bf16*>(p.o) + (int64_t)b * p.o_sb + (int64_t)qtok * p.o_sn + (int64_t)h * p.o_sh +
                lane * kPer;
#pragma unroll
  for (int e = 0; e < kPer; ++e) dst[e] = (__bf16)(acc[e] * inv);
  if (lane == 0)
    p.lse[((int64_t)b * p.Hq + h) * p.Nq + qtok] = L > 0.f ? (M + __log2f(L)) * 0.693147180559945309f : kNegInf;
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  const int64_t items = (int64_t)p.B * p.Hkv * p.n_qtiles;
  if (items == 0) return hipSuccess;
  const int64_t nwork = items * p.n_splits;
  if (p.kperm)
    hipLaunchKernelGGL((fwd_decode_kernel<D, true>), dim3((unsigned)nwork), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_decode_kernel<D, false>), dim3((unsigned)nwork), dim3(256), 0, stream, p);
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(items * 8)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t stream) {
  return d == 128 ? launch_decode_d<128>(p, stream) : launch_decode_d<64>(p, stream);
}

// Partial softmax states for bsattn_fwd_decode_noalloc, whose callers cannot allocate device
// memory: a buffer in the library's own device data.  Every GPU the library runs on holds its
// own copy until the process ends; in host code the name is only a host-side stand-in, so the
// kernels get the device address looked up below.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

// Device address of the current GPU's scratch array: looked up on the first call on each
// device (that device current) and kept per device.
hipError_t decode_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  *bytes = kDecodeScratchBytes;
  return hipSuccess;
}

}  // namespace bsattn
