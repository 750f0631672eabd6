// Page lists rebuilt on the device from a device-resident block selection (a selection that
// changes every step, e.g. the chunks chosen by bsattn_chunk_select), without a host round
// trip; the backward's transposed lists are rebuilt after them.  The rules are the host planner's: each (unit, Q block) row lists the pages of its
// selected K blocks, blocks ascending, pages ascending, packed as (first slot << 5) | valid
// rows, and every 4-entry stage (from the row's start) that holds a partial page or is cut
// short by the row's end carries bit 31 (KPage abstract, zhuanzhiai page 1, sentences 2 and
// 4).  Four small kernels: page counts per row, a prefix sum into the row pointers (clamped
// to the entry capacity), the entries, the stage flags; a wave per row, or a workgroup per
// row when the rows are fewer than the CUs.  Long count arrays are scanned over the whole
// chip, with the tile totals kept at the start of the entry array until the fill overwrites
// it (every reader masks entries past a list's end, so what they leave there is never used).
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

// The same counts for plans with few long rows (fewer rows than CUs, e.g. one Q block per
// sequence and KV group over thousands of chunks): a 1024-thread workgroup per row.
__global__ void __launch_bounds__(1024) plan_count_wide_kernel(PlanUpdateParams p) {
  __shared__ int64_t part[16];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j0 = p.row_ptr[r], j1 = p.row_ptr[r + 1];
  int64_t n = 0;
  for (int j = j0 + tid; j < j1; j += 1024) {
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
  if (lane == 0) part[w] = n;
  __syncthreads();
  if (tid == 0) {
    int64_t t = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) t += part[i];
    p.pl_ptr[r + 1] = (int32_t)(t < 0x7fffffff ? t : 0x7fffffff);
  }
}

// exclusive prefix sum of the counts, clamped to the capacity (one workgroup).  A tile of
// 16384 counts is four groups of 4096; in each group a thread takes four consecutive counts
// (every load and store instruction covers 1 KB), the groups are scanned within each wave by
// shuffles, and one 64-lane scan in wave 0 orders the 4 x 16 wave totals (lane 16 h + w:
// group h, wave w).  The running total is carried from tile to tile.
__global__ void __launch_bounds__(1024) plan_scan_kernel(PlanUpdateParams p) {
  constexpr int kGroups = 4, kTile = 4096 * kGroups;
  __shared__ int64_t wsum[64];
  __shared__ int64_t s_tot;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int64_t carry = 0;
  for (int64_t base = 0; base < p.n_rows; base += kTile) {
    int32_t v[kGroups][4];
    int64_t tot[kGroups], incl[kGroups];
    // unconditional loads (slots past the end read the last count and are zeroed), so that
    // all sixteen are in flight together instead of one branch and one wait each
#pragma unroll
    for (int h = 0; h < kGroups; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = base + 4096 * h + 4 * tid + i;
        const int32_t x = p.pl_ptr[(r < p.n_rows ? r : p.n_rows - 1) + 1];
        v[h][i] = r < p.n_rows ? x : 0;
      }
    }
#pragma unroll
    for (int h = 0; h < kGroups; ++h) {
      tot[h] = (int64_t)v[h][0] + v[h][1] + v[h][2] + v[h][3];
      incl[h] = tot[h];
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
      for (int h = 0; h < kGroups; ++h) {
        const int64_t x = __shfl_up(incl[h], d, 64);
        if (lane >= d) incl[h] += x;
      }
    }
    if (lane == 63) {
#pragma unroll
      for (int h = 0; h < kGroups; ++h) wsum[16 * h + w] = incl[h];
    }
    __syncthreads();
    if (w == 0) {
      const int64_t x = wsum[lane];
      int64_t xi = x;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int64_t y = __shfl_up(xi, d, 64);
        if (lane >= d) xi += y;
      }
      wsum[lane] = xi - x;  // exclusive offsets of (group, wave)
      if (lane == 63) s_tot = xi;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kGroups; ++h) {
      int64_t run = carry + wsum[16 * h + w] + incl[h] - tot[h];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = base + 4096 * h + 4 * tid + i;
        run += v[h][i];
        if (r < p.n_rows) p.pl_ptr[r + 1] = (int32_t)(run < p.capacity ? run : p.capacity);
      }
    }
    carry += s_tot;
    __syncthreads();  // wsum and s_tot are rewritten by the next tile
  }
  if (tid == 0) {
    p.pl_ptr[0] = 0;
    if (carry > p.capacity) flag(p, 1);
  }
}

// The same scan over the whole chip, for count arrays longer than one tile of the kernel
// above: the totals of 4096-count tiles (plan_tile_sum_kernel), their exclusive scan in one
// workgroup (plan_tile_scan_kernel), then each tile's own scan from its offset
// (plan_tile_apply_kernel).  The tile totals live at the start of the entry array, which
// only the fill writes, after the scan.
__device__ __forceinline__ int32_t count_at(const PlanUpdateParams& p, int64_t r) {
  const int32_t x = p.pl_ptr[(r < p.n_rows ? r : p.n_rows - 1) + 1];  // unconditional load
  return r < p.n_rows ? x : 0;
}

__global__ void __launch_bounds__(1024) plan_tile_sum_kernel(PlanUpdateParams p, int64_t* tsum) {
  __shared__ int64_t part[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t base = (int64_t)blockIdx.x * 4096 + 4 * tid;
  int64_t t = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) t += count_at(p, base + i);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) t += __shfl_xor(t, m, 64);
  if (lane == 0) part[w] = t;
  __syncthreads();
  if (tid == 0) {
    int64_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += part[i];
    tsum[blockIdx.x] = s;
  }
}

__global__ void __launch_bounds__(1024) plan_tile_scan_kernel(int64_t* tsum, int n_tiles) {
  __shared__ int64_t wsum[16];
  __shared__ int64_t s_tot;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int64_t carry = 0;
  for (int base = 0; base < n_tiles; base += 1024) {
    const int i = base + tid;
    const int64_t x = i < n_tiles ? tsum[i] : 0;
    int64_t incl = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (w == 0) {
      const int64_t y = lane < 16 ? wsum[lane] : 0;
      int64_t yi = y;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) {
        const int64_t z = __shfl_up(yi, d, 64);
        if (lane >= d) yi += z;
      }
      if (lane < 16) wsum[lane] = yi - y;
      if (lane == 15) s_tot = yi;
    }
    __syncthreads();
    if (i < n_tiles) tsum[i] = carry + wsum[w] + incl - x;  // exclusive tile offsets
    carry += s_tot;
    __syncthreads();
  }
}

__global__ void __launch_bounds__(1024) plan_tile_apply_kernel(PlanUpdateParams p, const int64_t* tsum, int n_tiles) {
  __shared__ int64_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t base = (int64_t)blockIdx.x * 4096 + 4 * tid;
  int32_t v[4];
  int64_t tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = count_at(p, base + i);
    tot += v[i];
  }
  int64_t incl = tot;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t x = __shfl_up(incl, d, 64);
    if (lane >= d) incl += x;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int64_t x = lane < 16 ? wsum[lane] : 0;
    int64_t xi = x;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int64_t y = __shfl_up(xi, d, 64);
      if (lane >= d) xi += y;
    }
    if (lane < 16) wsum[lane] = xi - x;
  }
  __syncthreads();
  int64_t run = tsum[blockIdx.x] + wsum[w] + incl - tot;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    run += v[i];
    if (base + i < p.n_rows) p.pl_ptr[base + i + 1] = (int32_t)(run < p.capacity ? run : p.capacity);
  }
  if ((int)blockIdx.x == n_tiles - 1 && tid == 1023 && run > p.capacity) flag(p, 1);  // run: the grand total
  if (blockIdx.x == 0 && tid == 0) p.pl_ptr[0] = 0;
}

// prefix sum of p's counts: the chip-wide form when the array spans more than one tile of
// plan_scan_kernel and the entry array (scratch, capacity entries) holds the tile totals
static void launch_scan(const PlanUpdateParams& p, int32_t* scratch, int64_t scratch_cap, hipStream_t stream) {
  const int64_t n_tiles = (int64_t(p.n_rows) + 4095) / 4096;
  if (p.n_rows > 16384 && (reinterpret_cast<uintptr_t>(scratch) & 7) == 0 && scratch_cap >= 2 * n_tiles) {
    int64_t* tsum = reinterpret_cast<int64_t*>(scratch);
    hipLaunchKernelGGL(plan_tile_sum_kernel, dim3((unsigned)n_tiles), dim3(1024), 0, stream, p, tsum);
    hipLaunchKernelGGL(plan_tile_scan_kernel, dim3(1), dim3(1024), 0, stream, tsum, (int)n_tiles);
    hipLaunchKernelGGL(plan_tile_apply_kernel, dim3((unsigned)n_tiles), dim3(1024), 0, stream, p,
                       (const int64_t*)tsum, (int)n_tiles);
  } else {
    hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, stream, p);
  }
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

// entries for plans with few long rows: a 1024-thread workgroup per row, threads over the
// row's blocks 1024 at a time, placed by a workgroup prefix sum (wave shuffles, then the 16
// wave totals through LDS)
__global__ void __launch_bounds__(1024) plan_fill_wide_kernel(PlanUpdateParams p) {
  __shared__ int wsum[16];
  __shared__ int s_tot;
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int base = p.pl_ptr[r], end = p.pl_ptr[r + 1];
  const int j0 = p.row_ptr[r], j1 = p.row_ptr[r + 1];
  int run = 0;
  for (int jb = j0; jb < j1; jb += 1024) {
    const int j = jb + tid;
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
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (w == 0) {
      const int x = lane < 16 ? wsum[lane] : 0;
      int xi = x;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) {
        const int y = __shfl_up(xi, d, 64);
        if (lane >= d) xi += y;
      }
      if (lane < 16) wsum[lane] = xi - x;  // exclusive wave offsets
      if (lane == 15) s_tot = xi;          // pages of these 1024 blocks
    }
    __syncthreads();
    const int pos0 = base + run + wsum[w] + incl - np;
    for (int i = 0; i < np; ++i) {
      const int pos = pos0 + i;
      if (pos < end) p.pl_ent[pos] = p.page_ent[p.first_page[kb] + i];
    }
    run += s_tot;
    __syncthreads();  // wsum and s_tot are rewritten by the next round
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

// stage flags for plans with few long rows: a 1024-thread workgroup per row
__global__ void __launch_bounds__(1024) plan_flag_wide_kernel(PlanUpdateParams p) {
  const int r = blockIdx.x;
  const int a = p.pl_ptr[r], b = p.pl_ptr[r + 1];
  for (int s0 = a + 4 * (int)threadIdx.x; s0 < b; s0 += 4096) {
    const int s1 = min(s0 + 4, b);
    bool partial = s1 - s0 < 4;
    for (int e = s0; e < s1; ++e) partial |= (p.pl_ent[e] & 31) < 16;
    if (partial)
      for (int e = s0; e < s1; ++e) p.pl_ent[e] = (int32_t)((uint32_t)p.pl_ent[e] | 0x80000000u);
  }
}

// ---------------------------------------------------------------------------------------
// Transposed lists for the backward: for each (unit, K block), the Q pages of every Q block
// whose selection row holds the K block -- Q blocks ascending, pages ascending -- the order
// the host planner uses, so the backward walks the same pairs in the same order.  A wave
// takes one list, its lanes test 64 Q blocks at a time (binary search in the block's
// ascending selection row), and a lane prefix sum places each member's pages.

// whether K block kb is in the ascending row kblk[a, b)
__device__ __forceinline__ bool row_has(const int32_t* kblk, int a, int b, int kb) {
  while (a < b) {
    const int m = (a + b) >> 1;
    const int v = kblk[m];
    if (v == kb) return true;
    if (v < kb) a = m + 1;
    else b = m;
  }
  return false;
}

// Q pages that list t = unit * nkb + kb receives from Q block qb (0 when qb does not select kb)
__device__ __forceinline__ int tpl_pages_of(const PlanUpdateParams& p, int t, int qb) {
  if (qb >= p.nqb) return 0;
  const int unit = t / p.nkb, kb = t - unit * p.nkb;
  const int row = unit * p.nqb + qb;
  return row_has(p.kblk, p.row_ptr[row], p.row_ptr[row + 1], kb) ? p.first_qpage[qb + 1] - p.first_qpage[qb] : 0;
}

// entries of each transposed list into tpl_ptr[t + 1]: one wave per list
__global__ void __launch_bounds__(256) tpl_count_kernel(PlanUpdateParams p) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= p.n_units * p.nkb) return;
  int64_t n = 0;
  for (int qb0 = 0; qb0 < p.nqb; qb0 += 64) n += tpl_pages_of(p, t, qb0 + lane);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) n += __shfl_xor(n, m, 64);
  if (lane == 0) p.tpl_ptr[t + 1] = (int32_t)(n < 0x7fffffff ? n : 0x7fffffff);
}

// the same with one thread per list, for plans of few Q blocks (a decode or prefill block
// per unit), where a wave per list would leave most lanes idle
__global__ void __launch_bounds__(256) tpl_count_small_kernel(PlanUpdateParams p) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= p.n_units * p.nkb) return;
  int64_t n = 0;
  for (int qb = 0; qb < p.nqb; ++qb) n += tpl_pages_of(p, t, qb);
  p.tpl_ptr[t + 1] = (int32_t)(n < 0x7fffffff ? n : 0x7fffffff);
}

__global__ void __launch_bounds__(256) tpl_fill_small_kernel(PlanUpdateParams p) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= p.n_units * p.nkb) return;
  const int base = p.tpl_ptr[t], end = p.tpl_ptr[t + 1];
  int pos = base;
  for (int qb = 0; qb < p.nqb; ++qb) {
    const int np = tpl_pages_of(p, t, qb);
    for (int i = 0; i < np; ++i, ++pos)
      if (pos < end) p.tpl_ent[pos] = p.qpage_ent[p.first_qpage[qb] + i];
  }
}

// the entries: one wave per list, lanes over its Q blocks 64 at a time
__global__ void __launch_bounds__(256) tpl_fill_kernel(PlanUpdateParams p) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= p.n_units * p.nkb) return;
  const int base = p.tpl_ptr[t], end = p.tpl_ptr[t + 1];
  int run = 0;
  for (int qb0 = 0; qb0 < p.nqb; qb0 += 64) {
    const int qb = qb0 + lane;
    const int np = tpl_pages_of(p, t, qb);
    int incl = np;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    const int pos0 = base + run + incl - np;
    for (int i = 0; i < np; ++i) {
      const int pos = pos0 + i;
      if (pos < end) p.tpl_ent[pos] = p.qpage_ent[p.first_qpage[qb] + i];
    }
    run += __shfl(incl, 63, 64);
  }
}

hipError_t launch_plan_update(const PlanUpdateParams& p, hipStream_t stream) {
  if (p.n_rows <= 0) return hipSuccess;
  if (p.n_rows < 256) {  // fewer rows than CUs: a workgroup per row
    hipLaunchKernelGGL(plan_count_wide_kernel, dim3(p.n_rows), dim3(1024), 0, stream, p);
    launch_scan(p, p.pl_ent, p.capacity, stream);
    hipLaunchKernelGGL(plan_fill_wide_kernel, dim3(p.n_rows), dim3(1024), 0, stream, p);
    hipLaunchKernelGGL(plan_flag_wide_kernel, dim3(p.n_rows), dim3(1024), 0, stream, p);
  } else {
    hipLaunchKernelGGL(plan_count_kernel, dim3((p.n_rows + 3) / 4), dim3(256), 0, stream, p);
    launch_scan(p, p.pl_ent, p.capacity, stream);
    hipLaunchKernelGGL(plan_fill_kernel, dim3((p.n_rows + 3) / 4), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(plan_flag_kernel, dim3((p.n_rows + 3) / 4), dim3(256), 0, stream, p);
  }
  const int64_t n_lists = int64_t(p.n_units) * p.nkb;
  if (p.tpl_ptr != nullptr && n_lists > 0) {
    // the transposed lists: count, prefix sum (the same scan, clamped to their capacity), fill
    PlanUpdateParams t = p;
    t.pl_ptr = p.tpl_ptr;
    t.n_rows = int32_t(n_lists);
    t.capacity = p.tcapacity;
    if (p.nqb <= 16) {
      const unsigned grid = (unsigned)((n_lists + 255) / 256);
      hipLaunchKernelGGL(tpl_count_small_kernel, dim3(grid), dim3(256), 0, stream, t);
      launch_scan(t, p.tpl_ent, p.tcapacity, stream);
      hipLaunchKernelGGL(tpl_fill_small_kernel, dim3(grid), dim3(256), 0, stream, t);
    } else {
      const unsigned grid = (unsigned)((n_lists + 3) / 4);
      hipLaunchKernelGGL(tpl_count_kernel, dim3(grid), dim3(256), 0, stream, t);
      launch_scan(t, p.tpl_ent, p.tcapacity, stream);
      hipLaunchKernelGGL(tpl_fill_kernel, dim3(grid), dim3(256), 0, stream, t);
    }
  }
  return hipGetLastError();
}

}  // namespace bsattn
