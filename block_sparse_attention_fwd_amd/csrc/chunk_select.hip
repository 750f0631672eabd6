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
// in LDS: a radix select of the topk-th key, then an ascending compaction.
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

constexpr int kMaxChunks = 8192;  // per (b, g): one 32-bit key per chunk in LDS

// top-k: one workgroup of 1024 threads per (b, g).  Each chunk gets the 32-bit key
// u = ~(order-preserving bits of its score), so ascending u is descending score, and the
// selection is the topk smallest (u, id) pairs: a radix select finds the topk-th smallest u
// (T) and how many chunks with u == T it takes (need); one scan in id order then writes the
// ids with u < T, and the first `need` ids with u == T, in ascending order.
template <int D>
__global__ void __launch_bounds__(1024) chunk_topk_kernel(ChunkParams p) {
  __shared__ float iq[D];
  __shared__ uint32_t uk[kMaxChunks];
  __shared__ int hist[256];
  __shared__ int wsum[16];
  __shared__ int pick[2];  // digit of the pass, chunks in the bins below it
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
  {
    constexpr int LPR = D / 4, RPI = 64 / LPR, U = 8;
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
        if (lane % LPR == 0 && c < n) {
          const uint32_t w = __float_as_uint(s[u]);
          uk[c] = ~((w >> 31) ? ~w : (w | 0x80000000u));
        }
      }
    }
  }
  __syncthreads();

  // radix select, 8 bits per pass from the top: among the keys that match the digits fixed
  // so far, the bin holding the kk-th smallest key fixes the next digit
  uint32_t prefix = 0, mask = 0;
  int kk = p.topk;  // rank (from 1) of the wanted key among the keys that match prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int c = tid; c < n; c += 1024) {
      const uint32_t u = uk[c];
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    if (wave == 0) {
      int h[4], loc = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[j] = hist[4 * lane + j];
        loc += h[j];
      }
      int inc = loc;  // inclusive scan over the wave's lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o, 64);
        inc += lane >= o ? v : 0;
      }
      int before = inc - loc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (before < kk && kk <= before + h[j]) {  // exactly one bin of the wave
          pick[0] = 4 * lane + j;
          pick[1] = before;
        }
        before += h[j];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)pick[0] << shift;
    mask |= 255u << shift;
    kk -= pick[1];
  }
  const uint32_t T = prefix;  // the topk-th smallest key
  const int need = kk;        // chunks with key T that are selected (1 .. count of them)

  // scan in id order: thread t owns ids [t per, (t + 1) per); counts of keys below T (low
  // 16 bits) and equal to T (high 16 bits), n <= 8192 so neither overflows
  const int per = (n + 1023) >> 10;
  const int c0 = min(n, tid * per), c1 = min(n, c0 + per);
  int loc = 0;
  for (int c = c0; c < c1; ++c) {
    const uint32_t u = uk[c];
    loc += (u < T ? 1 : 0) + (u == T ? 0x10000 : 0);
  }
  int inc = loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, 64);
    inc += lane >= o ? v : 0;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int pre = inc - loc;
  for (int w = 0; w < wave; ++w) pre += wsum[w];
  int lt = pre & 0xffff, eq = pre >> 16;
  int32_t* out = p.chunks + (int64_t)bg * p.topk;
  for (int c = c0; c < c1; ++c) {
    const uint32_t u = uk[c];
    if (u < T) {
      out[lt + min(eq, need)] = c;
      ++lt;
    } else if (u == T) {
      if (eq < need) out[lt + eq] = c;
      ++eq;
    }
  }
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
