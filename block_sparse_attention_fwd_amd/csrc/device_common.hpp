// Device helpers shared by the forward and backward kernels: vector types, scalar-load
// vectors, address spaces, page-list entry fields, wait counters, the LDS row swizzle
// and cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

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

// Page-list entry word: valid rows in bits 0..4, first slot in bits 5..30, and bit 31 set on
// the entries of a 4-entry stage that holds a partial page or ends past its list.
__device__ __forceinline__ int ent_nv(int ent) { return ent & 31; }
__device__ __forceinline__ int ent_slot(int ent) { return (ent >> 5) & ((1 << 26) - 1); }
constexpr float kLn2 = 0.693147180559945309f;

// Ties a register value to this point of the program: an empty asm statement that uses it.
// Device pass only (the host pass instantiates kernels for their launch stubs, and "v" names
// no host register class).
template <typename T>
__device__ __forceinline__ void pin(const T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#endif
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};
template <int I>
struct IntTag {
  static constexpr int value = I;
};
// f(IntTag<I>{}) for I = B .. E - 1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntTag<B>{});
    static_for<B + 1, E>(f);
  }
}

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
__device__ __forceinline__ float sum16v(const f32x16& x) {
  const float a = (x[0] + x[1]) + (x[2] + x[3]), b2 = (x[4] + x[5]) + (x[6] + x[7]);
  const float c = (x[8] + x[9]) + (x[10] + x[11]), d = (x[12] + x[13]) + (x[14] + x[15]);
  return (a + b2) + (c + d);
}

}  // namespace bsattn
