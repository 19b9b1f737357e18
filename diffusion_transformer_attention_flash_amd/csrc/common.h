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

// Workspace of the grid-wide reductions: per-workgroup partials of their
// fixed grids (kRedBlocks partial maxima per tensor for the fp8 amax, or
// kResBlocks float64 pairs for the residual sums), then, at kCounterOffset,
// the residual sums' arrival counters: one top counter and kResGroups group
// counters, each on its own 256-byte line. The counters must be zero before
// a call and are zero again after it.
constexpr int kRedBlocks = 1024;
constexpr int kResBlocks = 512;
constexpr int kResGroups = 16;
constexpr size_t kCounterOffset = 16384;
constexpr size_t kWsBytes = kCounterOffset + 256 * (1 + kResGroups);
static_assert(sizeof(double) * 2 * kResBlocks <= kCounterOffset, "residual partials fit");
static_assert(kResBlocks % kResGroups == 0, "equal groups");

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

// The extra-barrier build (-DDTA_DEBUG_BARRIERS): a workgroup barrier at every
// point where an attention kernel hands LDS from one phase to the next, on top
// of the synchronisation the kernels rely on. Its outputs must not change.
#ifndef DTA_DEBUG_BARRIERS
#define DTA_DEBUG_BARRIERS 0
#endif
constexpr bool kDebugBarriers = DTA_DEBUG_BARRIERS != 0;
__device__ __forceinline__ void debug_sync() {
  if constexpr (kDebugBarriers) __syncthreads();
}

// Orders a wave's LDS writes before its later LDS reads of cells that other
// lanes of the same wave wrote (wavefront scope: no s_barrier; LDS
// instructions of one wave complete in order, so this only stops the
// compiler from moving the accesses across it).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
