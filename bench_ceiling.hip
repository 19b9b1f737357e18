// Read-only HBM scan of a known byte count: the bandwidth ceiling bench.py
// sets beside the bandwidth-bound kernels of the library (residual_diff
// reads 56.6 MB and writes a few bytes). Not part of the library.
//
// Each thread xor-folds 16-byte chunks, U of them in flight per grid-stride
// step; a workgroup stores its fold only if it equals an arbitrary tag, so the
// loads are live but the stores (almost) never happen.

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void scan_kernel(const u32x4* __restrict__ x, int64_t n16,
                                                   uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = x[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = x[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;
}

// x: device buffer of `bytes` bytes (a multiple of 16, 16-byte aligned);
// out: device uint32[grid]; unroll in {1, 2, 4, 8}. Returns 0 or -1.
extern "C" int scan_read_only(const void* x, int64_t bytes, void* out, int grid, int unroll,
                              hipStream_t stream) {
  if (!x || !out || bytes < 16 || (bytes & 15) || grid < 1 ||
      (reinterpret_cast<uintptr_t>(x) & 15))
    return -1;
  const u32x4* p = static_cast<const u32x4*>(x);
  uint32_t* o = static_cast<uint32_t*>(out);
  const int64_t n16 = bytes >> 4;
  switch (unroll) {
    case 1: hipLaunchKernelGGL(scan_kernel<1>, dim3(grid), dim3(256), 0, stream, p, n16, o); break;
    case 2: hipLaunchKernelGGL(scan_kernel<2>, dim3(grid), dim3(256), 0, stream, p, n16, o); break;
    case 4: hipLaunchKernelGGL(scan_kernel<4>, dim3(grid), dim3(256), 0, stream, p, n16, o); break;
    case 8: hipLaunchKernelGGL(scan_kernel<8>, dim3(grid), dim3(256), 0, stream, p, n16, o); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
