// Dense-MFMA calibration for gfx950 (MI355X): the rate the matrix cores sustain on the
// forward's product, v_mfma_f32_32x32x16_bf16, with nothing else running.
//
// Every wave keeps eight A and four B operands in registers and issues 32 products per
// iteration into four independent accumulators, so the loop has no memory traffic and no
// dependency stall; with two workgroups of four waves per CU every SIMD holds two waves.
// The operands are pseudo-random bf16 values with a unit-normal-like spread (sums of six
// uniforms from a counter hash) or zeros: under the chip's power limit the sustained clock,
// and with it the rate, depends on how many operand bits toggle.  The first wave of each
// workgroup records the spans of the shader-clock counter (s_memtime) and of the 100 MHz
// real-time counter (s_memrealtime) around its loop, from which the caller derives the
// mean shader clock.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.hpp"

namespace bsattn {

__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// a bf16 value of mean 0 and variance about 1: six 16-bit uniforms summed, centred, scaled
__device__ __forceinline__ __bf16 probe_value(uint32_t seed) {
  const uint32_t a = probe_hash(seed), b = probe_hash(seed ^ 0x9e3779b9u), c = probe_hash(seed * 3u + 7u);
  const float u = (float)((a & 0xffffu) + (a >> 16) + (b & 0xffffu) + (b >> 16) + (c & 0xffffu) + (c >> 16)) / 65536.f;
  return (__bf16)((u - 3.f) * 1.41f);
}

__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, int random, uint64_t* clocks) {
  const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
  bf16x8 A[8], B[4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) A[i][e] = random ? probe_value(tid * 131u + i * 8 + e) : (__bf16)0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) B[i][e] = random ? probe_value(tid * 977u + 1000u + i * 8 + e) : (__bf16)0.f;
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], B[j], acc[j], 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[j][e];
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
  // keeps the products live: a sum that is never exactly this value on real data
  if (sum == 1.2345678e30f) clocks[2 * blockIdx.x] = 0;
}

hipError_t launch_mfma_probe(int n_workgroups, int iters, int random, uint64_t* clocks, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(n_workgroups), dim3(256), 0, stream, iters, random, clocks);
  return hipGetLastError();
}

}  // namespace bsattn
