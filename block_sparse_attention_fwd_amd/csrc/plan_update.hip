// Page lists rebuilt on the device from a device-resident block selection (a selection that
// changes every step, e.g. the chunks chosen by bsattn_chunk_select), without a host round
// trip.  The rules are the host planner's: each (unit, Q block) row lists the pages of its
// selected K blocks, blocks ascending, pages ascending, packed as (first slot << 5) | valid
// rows, and every 4-entry stage (from the row's start) that holds a partial page or is cut
// short by the row's end carries bit 31 (KPage abstract, zhuanzhiai page 1, sentences 2 and
// 4).  Four small kernels: page counts per row, a prefix sum into the row pointers (clamped
// to the entry capacity), the entries, the stage flags.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_params.hpp"

namespace bsattn {

__device__ __forceinline__ void flag(const PlanUpdateParams& p, int bit) {
  if (p.status) atomicOr(p.status, bit);
}

// pages of each row into pl_ptr[r + 1]: one wave per row, lanes over its blocks
__global__ void __launch_bounds__(256) plan_count_kernel(PlanUpdateParams p) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= p.n_rows) return;
  const int j0 = p.row_ptr[r], j1 = p.row_ptr[r + 1];
  int64_t n = 0;
  for (int j = j0 + lane; j < j1; j += 64) {
    const int kb = p.kblk[j];
    if (kb < 0 || kb >= p.nkb) {
      flag(p, 2);
      continue;
    }
    if (j > j0 && kb <= p.kblk[j - 1]) flag(p, 4);
    n += p.first_page[kb + 1] - p.first_page[kb];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) n += __shfl_xor(n, m, 64);
  if (lane == 0) p.pl_ptr[r + 1] = (int32_t)(n < 0x7fffffff ? n : 0x7fffffff);
}

// exclusive prefix sum of the counts, clamped to the capacity (one workgroup)
__global__ void __launch_bounds__(1024) plan_scan_kernel(PlanUpdateParams p) {
  __shared__ int64_t part[1024];
  const int tid = threadIdx.x;
  const int per = (p.n_rows + 1023) / 1024;
  const int r0 = min(p.n_rows, tid * per), r1 = min(p.n_rows, r0 + per);
  int64_t local = 0;
  for (int r = r0; r < r1; ++r) local += p.pl_ptr[r + 1];
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int64_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int64_t run = part[tid] - local;
  for (int r = r0; r < r1; ++r) {
    run += p.pl_ptr[r + 1];
    p.pl_ptr[r + 1] = (int32_t)(run < p.capacity ? run : p.capacity);
  }
  if (tid == 0) p.pl_ptr[0] = 0;
  if (tid == 1023 && part[1023] > p.capacity) flag(p, 1);
}

// entries: one wave per row, lanes over the row's blocks 64 at a time
__global__ void __launch_bounds__(256) plan_fill_kernel(PlanUpdateParams p) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= p.n_rows) return;
  const int base = p.pl_ptr[r], end = p.pl_ptr[r + 1];
  const int j0 = p.row_ptr[r], j1 = p.row_ptr[r + 1];
  int run = 0;
  for (int jb = j0; jb < j1; jb += 64) {
    const int j = jb + lane;
    int kb = -1, np = 0;
    if (j < j1) {
      kb = p.kblk[j];
      if (kb >= 0 && kb < p.nkb) np = p.first_page[kb + 1] - p.first_page[kb];
    }
    int incl = np;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    const int pos0 = base + run + incl - np;
    for (int i = 0; i < np; ++i) {
      const int pos = pos0 + i;
      if (pos < end) p.pl_ent[pos] = p.page_ent[p.first_page[kb] + i];
    }
    run += __shfl(incl, 63, 64);
  }
}

// stage flags: one wave per row, lanes over its 4-entry stages
__global__ void __launch_bounds__(256) plan_flag_kernel(PlanUpdateParams p) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= p.n_rows) return;
  const int a = p.pl_ptr[r], b = p.pl_ptr[r + 1];
  for (int s0 = a + 4 * lane; s0 < b; s0 += 256) {
    const int s1 = min(s0 + 4, b);
    bool partial = s1 - s0 < 4;
    for (int e = s0; e < s1; ++e) partial |= (p.pl_ent[e] & 31) < 16;
    if (partial)
      for (int e = s0; e < s1; ++e) p.pl_ent[e] = (int32_t)((uint32_t)p.pl_ent[e] | 0x80000000u);
  }
}

hipError_t launch_plan_update(const PlanUpdateParams& p, hipStream_t stream) {
  if (p.n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(plan_count_kernel, dim3((p.n_rows + 3) / 4), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, stream, p);
  hipLaunchKernelGGL(plan_fill_kernel, dim3((p.n_rows + 3) / 4), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(plan_flag_kernel, dim3((p.n_rows + 3) / 4), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace bsattn
