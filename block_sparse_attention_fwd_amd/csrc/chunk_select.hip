// Chunk selection for chunk-indexed sparse attention on gfx950 (MI355X).
//
// CISA abstract (fugumt page 4), sentences 3-5: fixed-size KV chunks are selected with
// compact summaries of the existing keys; one indexing query per KV group scores them and
// the selected chunks are shared by the group's queries.  Here:
//   summary[b, g, c] = mean of the keys of chunk c (chunk consecutive tokens, the last
//                      chunk may be short), fp32                     (chunk_summary_kernel)
//   iq[b, g]         = mean over the group's query heads of Q at row query_index
//   score[b, g, c]   = <summary, iq>; the topk best chunks, ties to the lower chunk id,
//                      listed in ascending order                       (chunk_topk_kernel)
// The summaries are the part CISA keeps between steps; they are an output.  Reading K once
// is the whole cost (HBM-bound); the selection itself works on n_chunks scores per (b, g)
// in LDS: a bitonic sort of (score, id) keys, then an ascending compaction.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.hpp"
#include "kernel_params.hpp"

namespace bsattn {

// summaries: one wave per (b, chunk, g), g fastest, so that the waves of a workgroup and
// neighbouring workgroups read adjacent head slices of the same key rows (whole rows of the
// usual [B, N, H, d] layout stream through together).  Lane (r, col) sums rows
// t = r (mod 64 / (D / 8)) of the chunk over 8 columns from 16-byte loads, four loads in
// flight per step; the row groups are then combined by shuffles.
template <int D>
__global__ void __launch_bounds__(256) chunk_summary_kernel(ChunkParams p) {
  constexpr int L = D / 8;     // lanes per row
  constexpr int RPI = 64 / L;  // rows per load instruction
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b * n_chunks + c) * Hkv + g
  if (item >= (int64_t)p.B * p.Hkv * p.n_chunks) return;  // whole waves leave together
  const int g = (int)(item % p.Hkv);
  const int64_t bc = item / p.Hkv;
  const int64_t b = bc / p.n_chunks;
  const int c = (int)(bc - b * p.n_chunks);
  const int t0 = c * p.chunk;
  const int t1 = min(p.Nk, t0 + p.chunk);
  const int col = (lane % L) * 8, r = lane / L;
  const __bf16* base = reinterpret_cast<const __bf16*>(p.k) + b * p.k_sb + g * p.k_sh + col;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int t = t0 + r;
  for (; t + 3 * RPI < t1; t += 4 * RPI) {
    bf16x8 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const bf16x8*>(base + (int64_t)(t + u * RPI) * p.k_sn);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (float)v[u][e];
  }
  for (; t < t1; t += RPI) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(base + (int64_t)t * p.k_sn);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
  }
#pragma unroll
  for (int m = L; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], m, 64);
  if (r == 0) {
    const float inv = 1.f / (float)(t1 - t0);
    float* dst = p.summ + ((b * p.Hkv + g) * p.n_chunks + c) * D + col;
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
}

constexpr int kMaxChunks = 8192;  // per (b, g): the sort keys fill 64 KB of LDS

// top-k: one workgroup of 1024 threads per (b, g)
template <int D>
__global__ void __launch_bounds__(1024) chunk_topk_kernel(ChunkParams p) {
  __shared__ float iq[D];
  __shared__ uint64_t keys[kMaxChunks];
  __shared__ int flag[kMaxChunks];
  __shared__ int cnt[1024];
  const int tid = threadIdx.x;
  const int bg = blockIdx.x;
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int n = p.n_chunks, npad = p.n_pad;

  if (tid < D) {
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb + (int64_t)p.query_index * p.q_sn +
                       (int64_t)(g * p.grp) * p.q_sh + tid;
    float s = 0.f;
    for (int h = 0; h < p.grp; ++h) s += (float)qp[(int64_t)h * p.q_sh];
    iq[tid] = s / (float)p.grp;
  }
  __syncthreads();
  // scores, coalesced: D/4 lanes read one summary row (16 bytes each) and reduce its dot
  // product by shuffles; every wave keeps U loads (U * 64 / (D / 4) rows) in flight.
  // key = (descending score, ascending id): ~(order-preserving score bits) << 32 | id
  {
    constexpr int LPR = D / 4, RPI = 64 / LPR, U = 8;
    const int lane = tid & 63, wave = tid >> 6;
    const int sub = lane / LPR, e0 = (lane % LPR) * 4;
    const float q0 = iq[e0], q1 = iq[e0 + 1], q2 = iq[e0 + 2], q3 = iq[e0 + 3];
    const float* srow = p.summ + (int64_t)bg * n * D + e0;
    for (int cb = wave * RPI * U; cb < npad; cb += 16 * RPI * U) {
      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = cb + u * RPI + sub;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c < n) v = *reinterpret_cast<const float4*>(srow + (int64_t)c * D);
        s[u] = __builtin_fmaf(v.w, q3, __builtin_fmaf(v.z, q2, __builtin_fmaf(v.y, q1, v.x * q0)));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) s[u] += __shfl_xor(s[u], m, 64);
        const int c = cb + u * RPI + sub;
        if (lane % LPR == 0 && c < npad) {
          uint64_t key = ~uint64_t(0);
          if (c < n) {
            const uint32_t w = __float_as_uint(s[u]);
            const uint32_t ord = (w >> 31) ? ~w : (w | 0x80000000u);
            key = (uint64_t(~ord) << 32) | uint32_t(c);
          }
          keys[c] = key;
        }
      }
    }
  }
  __syncthreads();
  // bitonic sort, ascending.  Element i of the network lives in LDS, except during the stages
  // whose partner distance j is below 64: then lane i % 64 of wave (i / 64) % 16 holds it in
  // register i / 1024 and takes the partner's key by a lane shuffle, so those stages need no
  // barrier (21 of the 78 stages of 4096 keys go through LDS).
  {
    constexpr int RMAX = kMaxChunks / 1024;
    const int nreg = npad >= 1024 ? npad / 1024 : 1;
    uint64_t a[RMAX];
    auto reg_load = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        const int i = tid + 1024 * r;
        if (r < nreg) a[r] = i < npad ? keys[i] : ~uint64_t(0);
      }
    };
    auto reg_store = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        const int i = tid + 1024 * r;
        if (r < nreg && i < npad) keys[i] = a[r];
      }
    };
    // every lane of the workgroup runs the shuffles (nreg is uniform); lanes past npad hold
    // dummies whose partners are dummies too (npad is a power of two and j < npad)
    auto reg_stage = [&](int k, int j) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        if (r < nreg) {
          const int i = tid + 1024 * r;
          const int lo = __shfl_xor((int)(uint32_t)a[r], j, 64);
          const int hi = __shfl_xor((int)(uint32_t)(a[r] >> 32), j, 64);
          const uint64_t o = (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
          const bool up = (i & k) == 0, lower = (i & j) == 0;
          const uint64_t mn = a[r] < o ? a[r] : o, mx = a[r] < o ? o : a[r];
          a[r] = lower == up ? mn : mx;
        }
      }
    };
    reg_load();
    for (int k = 2; k <= min(64, npad); k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) reg_stage(k, j);
    reg_store();
    __syncthreads();
    for (int k = 128; k <= npad; k <<= 1) {
      for (int j = k >> 1; j >= 64; j >>= 1) {
        for (int i = tid; i < npad; i += 1024) {
          const int l = i ^ j;
          if (l > i) {
            const uint64_t x = keys[i], y = keys[l];
            const bool up = (i & k) == 0;
            if ((x > y) == up) {
              keys[i] = y;
              keys[l] = x;
            }
          }
        }
        __syncthreads();
      }
      reg_load();
      for (int j = 32; j > 0; j >>= 1) reg_stage(k, j);
      reg_store();
      __syncthreads();
    }
  }
  // the first topk keys are the selection; list their ids in ascending order
  for (int c = tid; c < n; c += 1024) flag[c] = 0;
  __syncthreads();
  for (int i = tid; i < p.topk; i += 1024) flag[(int)(uint32_t)keys[i]] = 1;
  __syncthreads();
  const int per = (n + 1023) / 1024;
  const int c0 = min(n, tid * per), c1 = min(n, c0 + per);
  int local = 0;
  for (int c = c0; c < c1; ++c) local += flag[c];
  cnt[tid] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan (Hillis-Steele)
    const int v = tid >= off ? cnt[tid - off] : 0;
    __syncthreads();
    cnt[tid] += v;
    __syncthreads();
  }
  int pos = cnt[tid] - local;
  int32_t* out = p.chunks + (int64_t)bg * p.topk;
  for (int c = c0; c < c1; ++c)
    if (flag[c]) out[pos++] = c;
}

hipError_t launch_chunk_select(const ChunkParams& p, hipStream_t stream) {
  const int64_t items = (int64_t)p.B * p.Hkv * p.n_chunks;
  const unsigned gs = (unsigned)((items + 3) / 4);
  if (p.d == 128) {
    hipLaunchKernelGGL((chunk_summary_kernel<128>), dim3(gs), dim3(256), 0, stream, p);
    hipLaunchKernelGGL((chunk_topk_kernel<128>), dim3(p.B * p.Hkv), dim3(1024), 0, stream, p);
  } else {
    hipLaunchKernelGGL((chunk_summary_kernel<64>), dim3(gs), dim3(256), 0, stream, p);
    hipLaunchKernelGGL((chunk_topk_kernel<64>), dim3(p.B * p.Hkv), dim3(1024), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace bsattn
