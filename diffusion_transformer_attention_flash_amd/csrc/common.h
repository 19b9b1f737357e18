// Shared device helpers for the gfx950 kernels of libdta.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dta.h"

namespace dta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Workspace of the two grid-wide reductions: one partial (two doubles) per
// workgroup of their fixed grid.
constexpr int kRedBlocks = 1024;
constexpr size_t kWsBytes = sizeof(double) * 2 * kRedBlocks;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float32 -> bf16, two values packed into one dword
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Wave64 reductions through DPP-free cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// Remap a linear workgroup id so that the workgroups the hardware places on
// one XCD (ids congruent mod 8) get consecutive logical ids: neighbouring
// query tiles of one head then run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks >> 3;
  if (bid >= per * 8) return bid;
  return (bid & 7) * per + (bid >> 3);
}

}  // namespace dta
