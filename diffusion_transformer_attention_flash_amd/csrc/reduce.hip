// Grid-wide reductions over bf16 tensors:
// * residual_diff -- First Block Cache's relative residual difference
//   sum|a-b| / sum|b| (ParaAttention guide, section "First Block Cache").
// * fbcache_step -- the same reduction, the cache decision diff < threshold
//   into a device flag, and the flag-guarded apply hidden += cached.
// * fp8_quant_rows_pow2 -- row-wise E4M3 quantisation with one power-of-two
//   scale per row (the same section's more accurate option).
// * fp8_quant_per_tensor -- per-tensor dynamic E4M3FN quantisation, scale
//   amax|x|/448 (ParaAttention guide, section "fp8 quantization"), and
//   fp8_quant_per_tensor_multi, the same for up to four tensors (Q, K, V) in
//   the same two launches.
//
// The two grid-wide reductions (residual sums, fp8 amax) are HBM-bound scans.
// A fixed grid strides over the tensor in 16-byte chunks (two chunks per
// thread per step, so that four 128-bit loads are in flight), reduces in
// registers, then across the wave and the workgroup.
// * Residual sums (kResBlocks workgroups): each workgroup publishes its
//   partial pair with device-scope stores (which complete only where every
//   XCD sees them, so no L2 writeback is needed), waits for them to
//   complete, then counts itself in with a device-scope atomic add on its
//   group's counter (kResGroups counters on separate lines: one counter
//   for all workgroups serialises their adds and cost 10 us). The last of a
//   group counts the group in on the top counter; the last of those sums all
//   partials with device-scope loads in a fixed order in float64, writes the
//   result and returns every counter it used to zero. One launch, and the
//   result does not depend on which workgroup finishes last.
// * fp8 amax: every workgroup of the following cast kernel combines the
//   partial maxima itself with an integer max (order-free); the kernel
//   boundary publishes them.
// Both are bitwise reproducible.

#include <algorithm>
#include <mutex>

#include "common.h"

namespace dta {

// Workgroup-wide sum of two floats; valid in thread 0.
__device__ __forceinline__ void block_sum2(float& x, float& y) {
  __shared__ float sx[4], sy[4];
  x = wave_sum(x);
  y = wave_sum(y);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sx[wave] = x;
    sy[wave] = y;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    x = (sx[0] + sx[1]) + (sx[2] + sx[3]);
    y = (sy[0] + sy[1]) + (sy[2] + sy[3]);
  }
}

__device__ __forceinline__ void abs_diff_acc(uint32_t a, uint32_t b, float& num,
                                             float& den) {
  const float a0 = bf16_bits_to_f32(a & 0xFFFF), a1 = bf16_bits_to_f32(a >> 16);
  const float b0 = bf16_bits_to_f32(b & 0xFFFF), b1 = bf16_bits_to_f32(b >> 16);
  num += fabsf(a0 - b0) + fabsf(a1 - b1);
  den += fabsf(b0) + fabsf(b1);
}

// Sum|a-b| and sum|b| per workgroup; the last workgroup to arrive finishes:
// out = float(sum num / sum den) (FBCACHE: also *use_cache = out < threshold,
// a NaN giving 0).
template <bool FBCACHE>
__global__ __launch_bounds__(256) void residual_diff_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ b, int64_t n,
    double* __restrict__ part, unsigned* __restrict__ counter, float* __restrict__ out,
    float threshold, int* __restrict__ use_cache) {
  const int64_t n8 = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * 256;
  const u32x4* a4 = reinterpret_cast<const u32x4*>(a);
  const u32x4* b4 = reinterpret_cast<const u32x4*>(b);
  float num = 0.f, den = 0.f;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + stride < n8; i += 2 * stride) {
    const u32x4 xa0 = a4[i], xb0 = b4[i];
    const u32x4 xa1 = a4[i + stride], xb1 = b4[i + stride];
#pragma unroll
    for (int e = 0; e < 4; ++e) abs_diff_acc(xa0[e], xb0[e], num, den);
#pragma unroll
    for (int e = 0; e < 4; ++e) abs_diff_acc(xa1[e], xb1[e], num, den);
  }
  if (i < n8) {
    const u32x4 xa = a4[i], xb = b4[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) abs_diff_acc(xa[e], xb[e], num, den);
  }
  // Tail of fewer than 8 elements: the first threads of workgroup 0.
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t t = (n8 << 3) + threadIdx.x;
    const float av = bf16_bits_to_f32(a[t]), bv = bf16_bits_to_f32(b[t]);
    num += fabsf(av - bv);
    den += fabsf(bv);
  }
  block_sum2(num, den);
  __shared__ bool last;
  if (threadIdx.x == 0) {
    __hip_atomic_store(&part[2 * blockIdx.x], (double)num, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&part[2 * blockIdx.x + 1], (double)den, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    // Both stores have completed at device scope before this workgroup is
    // counted: whoever counts last then reads them.
    __builtin_amdgcn_s_waitcnt(0);
    constexpr unsigned kPer = kResBlocks / kResGroups;
    unsigned* group = counter + 64 * (1 + blockIdx.x % kResGroups);
    bool l = false;
    if (__hip_atomic_fetch_add(group, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        kPer - 1) {
      // Every workgroup of the group has counted in: reset its counter for
      // the next call and count the group in.
      __hip_atomic_store(group, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      l = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
          kResGroups - 1;
    }
    last = l;
  }
  __syncthreads();
  if (!last) return;
  // Fixed-order float64 sum of the partial pairs: thread t adds partials t,
  // t+256, ..., then a fixed binary tree.
  __shared__ double fx[256], fy[256];
  double x = 0.0, y = 0.0;
  for (int p = threadIdx.x; p < (int)gridDim.x; p += 256) {
    x += __hip_atomic_load(&part[2 * p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    y += __hip_atomic_load(&part[2 * p + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  fx[threadIdx.x] = x;
  fy[threadIdx.x] = y;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      fx[threadIdx.x] += fx[threadIdx.x + s];
      fy[threadIdx.x] += fy[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float d = (float)(fx[0] / fy[0]);
    *out = d;
    if constexpr (FBCACHE) *use_cache = (d < threshold) ? 1 : 0;
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// hidden += cached (float32 sum of two bf16, rounded once to bf16) when the
// flag is set; every workgroup leaves at once otherwise.
__global__ __launch_bounds__(256) void fbcache_apply_kernel(
    uint16_t* __restrict__ hidden, const uint16_t* __restrict__ cached, int64_t n,
    const int* __restrict__ use_cache) {
  if (*use_cache == 0) return;
  const int64_t n8 = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * 256;
  u32x4* h4 = reinterpret_cast<u32x4*>(hidden);
  const u32x4* c4 = reinterpret_cast<const u32x4*>(cached);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    const u32x4 h = h4[i], c = c4[i];
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r[e] = pack_bf16x2(bf16_bits_to_f32(h[e] & 0xFFFF) + bf16_bits_to_f32(c[e] & 0xFFFF),
                         bf16_bits_to_f32(h[e] >> 16) + bf16_bits_to_f32(c[e] >> 16));
    h4[i] = r;
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t t = (n8 << 3) + threadIdx.x;
    const float v = bf16_bits_to_f32(hidden[t]) + bf16_bits_to_f32(cached[t]);
    hidden[t] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFF);
  }
}

// |x| maximum over bf16 bit patterns: for non-NaN values the order of the
// sign-cleared 15-bit patterns is the order of the magnitudes.
__device__ __forceinline__ uint32_t amax_bits(uint32_t w, uint32_t m) {
  return max(m, max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
}

// Up to kQuantMax tensors of one per-tensor quantisation call. Workgroups
// are assigned tensor by tensor: blocks [t * per, (t + 1) * per) serve tensor
// t, so every tensor keeps the grid a single-tensor call would use.
constexpr int kQuantMax = 4;
static_assert(kQuantMax * kRedBlocks * sizeof(uint32_t) <= kCounterOffset,
              "amax partials fit ws below the residual counter");
struct QuantTable {
  const uint16_t* x[kQuantMax];
  uint8_t* x8[kQuantMax];
  int64_t n[kQuantMax];
};

__global__ __launch_bounds__(256) void amax_kernel(QuantTable tab, uint32_t* __restrict__ part) {
  const int ti = blockIdx.x / kRedBlocks, lb = blockIdx.x - ti * kRedBlocks;
  const uint16_t* __restrict__ x = tab.x[ti];
  const int64_t n = tab.n[ti];
  const int64_t n8 = n >> 3;
  const int64_t stride = (int64_t)kRedBlocks * 256;
  const u32x4* x4 = reinterpret_cast<const u32x4*>(x);
  uint32_t m = 0;
  int64_t i = (int64_t)lb * 256 + threadIdx.x;
  for (; i + stride < n8; i += 2 * stride) {
    const u32x4 v0 = x4[i], v1 = x4[i + stride];
#pragma unroll
    for (int e = 0; e < 4; ++e) m = amax_bits(v0[e], amax_bits(v1[e], m));
  }
  if (i < n8) {
    const u32x4 v0 = x4[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) m = amax_bits(v0[e], m);
  }
  if (lb == 0 && threadIdx.x < (n & 7))
    m = max(m, (uint32_t)(x[(n8 << 3) + threadIdx.x] & 0x7FFFu));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  __shared__ uint32_t sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t bm = max(max(sm[0], sm[1]), max(sm[2], sm[3]));
    part[ti * kRedBlocks + lb] = bm;
  }
}

// E4M3FN code of x / s: correctly rounded float32 division, clamp to the
// finite range, then v_cvt_pk_fp8_f32 (round to nearest even).
__device__ __forceinline__ float fp8_in(float x, float s) {
  return fminf(fmaxf(__fdiv_rn(x, s), -448.0f), 448.0f);
}

// Every workgroup first reduces its tensor's kRedBlocks partial maxima itself
// (one 16-byte load per thread, from L2) instead of a one-workgroup finish
// launch; the first workgroup of each tensor publishes that tensor's scale.
// Workgroups [t * per, (t + 1) * per) cast tensor t.
__global__ __launch_bounds__(256) void fp8_cast_kernel(
    QuantTable tab, int per, const uint32_t* __restrict__ part, float* __restrict__ descale) {
  static_assert(kRedBlocks == 4 * 256, "one 16-byte load of partials per thread");
  const int ti = blockIdx.x / per, lb = blockIdx.x - ti * per;
  __shared__ uint32_t sm[4];
  __shared__ float s_sh;
  {
    const u32x4 pv = reinterpret_cast<const u32x4*>(part + ti * kRedBlocks)[threadIdx.x];
    uint32_t r = max(max(pv[0], pv[1]), max(pv[2], pv[3]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) r = max(r, (uint32_t)__shfl_xor((int)r, off, 64));
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = r;
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t bm = max(max(sm[0], sm[1]), max(sm[2], sm[3]));
      const float amax = bf16_bits_to_f32(bm);
      const float sc = (amax == 0.f) ? 1.0f : __fdiv_rn(amax, 448.0f);
      s_sh = sc;
      if (lb == 0) descale[ti] = sc;
    }
    __syncthreads();
  }
  const float s = s_sh;
  const uint16_t* __restrict__ x = tab.x[ti];
  uint8_t* __restrict__ x8 = tab.x8[ti];
  const int64_t n = tab.n[ti];
  const int64_t n8 = n >> 3;
  const int64_t stride = (int64_t)per * 256;
  const u32x4* x4 = reinterpret_cast<const u32x4*>(x);
  for (int64_t i = (int64_t)lb * 256 + threadIdx.x; i < n8; i += stride) {
    const u32x4 v = x4[i];
    u32x2 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t lo = v[2 * h], hi = v[2 * h + 1];
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(
          fp8_in(bf16_bits_to_f32(lo & 0xFFFF), s),
          fp8_in(bf16_bits_to_f32(lo >> 16), s), 0, false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(
          fp8_in(bf16_bits_to_f32(hi & 0xFFFF), s),
          fp8_in(bf16_bits_to_f32(hi >> 16), s), wd, true);
      r[h] = (uint32_t)wd;
    }
    *reinterpret_cast<u32x2*>(x8 + i * 8) = r;
  }
  if (lb == 0 && threadIdx.x < (n & 7)) {
    const int64_t t = (n8 << 3) + threadIdx.x;
    const float y = fp8_in(bf16_bits_to_f32(x[t]), s);
    x8[t] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false) & 0xFF);
  }
}

// Row-wise power-of-two E4M3 quantisation: one 16-lane group per row of
// row_len (a multiple of 8) elements, 16-byte chunks. The exponent is the
// smallest e with amax <= 448 * 2^e, read off the bf16 bits of amax exactly:
// amax = (1 + f/128) 2^(E-127) is <= 448 * 2^e = 1.75 * 2^(8+e) iff
// e >= E-135 when f <= 96 (1 + f/128 <= 1.75), else e >= E-134. Scaling by
// 2^-e is exact (v_ldexp), then saturating RNE conversion.
__global__ __launch_bounds__(256) void fp8_rows_pow2_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int row_len, uint8_t* __restrict__ x8,
    uint8_t* __restrict__ e8m0) {
  const int grp = threadIdx.x >> 4, l16 = threadIdx.x & 15;
  const int cpr = row_len >> 3;
  for (int64_t r = (int64_t)blockIdx.x * 16 + grp; r < rows; r += (int64_t)gridDim.x * 16) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + r * row_len);
    uint32_t m = 0;
    for (int c = l16; c < cpr; c += 16) {
      const u32x4 v = xr[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) m = amax_bits(v[e], m);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 16));
    int ex = 0;
    if (m != 0) {
      const int E = (int)(m >> 7), f = (int)(m & 0x7F);
      ex = (f <= 96) ? E - 135 : E - 134;
      ex = max(ex, -127);
    }
    const float s = __builtin_ldexpf(1.0f, -ex);
    uint8_t* out = x8 + r * row_len;
    for (int c = l16; c < cpr; c += 16) {
      const u32x4 v = xr[c];
      u32x2 w;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t lo = v[2 * h], hi = v[2 * h + 1];
        auto y = [&](uint32_t b) {
          return fminf(fmaxf(bf16_bits_to_f32(b) * s, -448.0f), 448.0f);
        };
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(y(lo & 0xFFFF), y(lo >> 16), 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(y(hi & 0xFFFF), y(hi >> 16), wd, true);
        w[h] = (uint32_t)wd;
      }
      *reinterpret_cast<u32x2*>(out + c * 8) = w;
    }
    if (l16 == 0) e8m0[r] = (uint8_t)(ex + 127);
  }
}

}  // namespace dta

using namespace dta;

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

extern "C" size_t dta_ws_bytes(void) { return kWsBytes; }

static unsigned* ws_counter(void* ws) {
  return reinterpret_cast<unsigned*>(static_cast<char*>(ws) + kCounterOffset);
}

// residual_diff_noalloc's scratch: the same partials and counters as a
// caller's workspace, in a file-scope device array (one copy per GPU, kept
// until the process ends). It is zero when the library loads, and every call
// returns its counters to zero. In host code `scratch` names a host-side
// stand-in, never the device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kWsBytes];

namespace {
constexpr int kMaxDevices = 64;
// Largest n of the scratch-backed entry point: the scratch holds the fixed
// grid's partials whatever n is; this bound keeps the 64-bit chunk index
// arithmetic exact.
constexpr int64_t kNoAllocMaxN = (int64_t)1 << 62;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device with that device current.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DTA_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return DTA_ELAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DTA_OK;
}
}  // namespace

extern "C" int residual_diff(const void* a, const void* b, int64_t n, float* out,
                             void* ws, hipStream_t stream) {
  if (!a || !b || !out || !ws || n < 1) return DTA_EINVAL;
  if (!al16(a) || !al16(b) || !al16(ws) || (reinterpret_cast<uintptr_t>(out) & 3))
    return DTA_EALIGN;
  hipLaunchKernelGGL(residual_diff_kernel<false>, dim3(kResBlocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), n,
                     static_cast<double*>(ws), ws_counter(ws), out, 0.0f, nullptr);
  return hipGetLastError() == hipSuccess ? DTA_OK : DTA_ELAUNCH;
}

extern "C" int residual_diff_noalloc(const void* a, const void* b, int64_t n, float* out,
                                     hipStream_t stream) {
  if (!a || !b || !out || n < 1) return DTA_EINVAL;
  if (n >= kNoAllocMaxN) return DTA_EINVAL;
  if (!al16(a) || !al16(b) || (reinterpret_cast<uintptr_t>(out) & 3)) return DTA_EALIGN;
  if (stream != nullptr) {
    int dev = -1, cur = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || hipGetDevice(&cur) != hipSuccess)
      return DTA_ELAUNCH;
    if (dev != cur) return DTA_EINVAL;
  }
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != DTA_OK) return st;
  hipLaunchKernelGGL(residual_diff_kernel<false>, dim3(kResBlocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), n,
                     static_cast<double*>(ws), ws_counter(ws), out, 0.0f, nullptr);
  return hipGetLastError() == hipSuccess ? DTA_OK : DTA_ELAUNCH;
}

extern "C" int fbcache_step(const void* r, const void* r_prev, int64_t n, float threshold,
                            void* hidden, const void* cached, int64_t n_hidden,
                            float* diff, int* use_cache, void* ws, hipStream_t stream) {
  if (!r || !r_prev || !hidden || !cached || !diff || !use_cache || !ws) return DTA_EINVAL;
  if (n < 1 || n_hidden < 1) return DTA_EINVAL;
  if (!al16(r) || !al16(r_prev) || !al16(hidden) || !al16(cached) || !al16(ws) ||
      (reinterpret_cast<uintptr_t>(diff) & 3) || (reinterpret_cast<uintptr_t>(use_cache) & 3))
    return DTA_EALIGN;
  hipLaunchKernelGGL(residual_diff_kernel<true>, dim3(kResBlocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(r), static_cast<const uint16_t*>(r_prev), n,
                     static_cast<double*>(ws), ws_counter(ws), diff, threshold, use_cache);
  if (hipGetLastError() != hipSuccess) return DTA_ELAUNCH;
  const int64_t want = ((n_hidden >> 3) + 255) / 256;
  const unsigned grid = (unsigned)(want < 1 ? 1 : (want < 8192 ? want : 8192));
  hipLaunchKernelGGL(fbcache_apply_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<uint16_t*>(hidden), static_cast<const uint16_t*>(cached),
                     n_hidden, use_cache);
  return hipGetLastError() == hipSuccess ? DTA_OK : DTA_ELAUNCH;
}

// Both per-tensor entry points: amax partials of every tensor in one launch,
// then every tensor's cast in one launch.
static int launch_quant(const QuantTable& tab, int count, float* descale, void* ws,
                        hipStream_t stream) {
  uint32_t* part = static_cast<uint32_t*>(ws);
  hipLaunchKernelGGL(amax_kernel, dim3(count * kRedBlocks), dim3(256), 0, stream, tab, part);
  if (hipGetLastError() != hipSuccess) return DTA_ELAUNCH;
  int64_t want = 1;
  for (int t = 0; t < count; ++t)
    want = std::max<int64_t>(want, ((tab.n[t] >> 3) + 255) / 256);
  const int per = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(fp8_cast_kernel, dim3(count * per), dim3(256), 0, stream, tab, per, part,
                     descale);
  return hipGetLastError() == hipSuccess ? DTA_OK : DTA_ELAUNCH;
}

extern "C" int fp8_quant_per_tensor(const void* x, int64_t n, void* x8,
                                    float* descale, void* ws, hipStream_t stream) {
  if (!x || !x8 || !descale || !ws || n < 1) return DTA_EINVAL;
  if (!al16(x) || !al16(x8) || !al16(ws) || (reinterpret_cast<uintptr_t>(descale) & 3))
    return DTA_EALIGN;
  QuantTable tab = {};
  tab.x[0] = static_cast<const uint16_t*>(x);
  tab.x8[0] = static_cast<uint8_t*>(x8);
  tab.n[0] = n;
  return launch_quant(tab, 1, descale, ws, stream);
}

extern "C" int fp8_quant_per_tensor_multi(int count, const void* const* x, const int64_t* n,
                                          void* const* x8, float* descale, void* ws,
                                          hipStream_t stream) {
  if (count < 1 || count > kQuantMax || !x || !n || !x8 || !descale || !ws) return DTA_EINVAL;
  QuantTable tab = {};
  for (int t = 0; t < count; ++t) {
    if (!x[t] || !x8[t] || n[t] < 1) return DTA_EINVAL;
    if (!al16(x[t]) || !al16(x8[t])) return DTA_EALIGN;
    tab.x[t] = static_cast<const uint16_t*>(x[t]);
    tab.x8[t] = static_cast<uint8_t*>(x8[t]);
    tab.n[t] = n[t];
  }
  if (!al16(ws) || (reinterpret_cast<uintptr_t>(descale) & 3)) return DTA_EALIGN;
  return launch_quant(tab, count, descale, ws, stream);
}

extern "C" int fp8_quant_rows_pow2(const void* x, int64_t rows, int row_len, void* x8,
                                   void* e8m0, hipStream_t stream) {
  if (!x || !x8 || !e8m0 || rows < 1 || row_len < 8 || (row_len & 7)) return DTA_EINVAL;
  if (!al16(x) || (reinterpret_cast<uintptr_t>(x8) & 7)) return DTA_EALIGN;
  const int64_t want = (rows + 15) / 16;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(fp8_rows_pow2_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), rows, row_len,
                     static_cast<uint8_t*>(x8), static_cast<uint8_t*>(e8m0));
  return hipGetLastError() == hipSuccess ? DTA_OK : DTA_ELAUNCH;
}

extern "C" const char* dta_status_str(int status) {
  switch (status) {
    case DTA_OK: return "ok";
    case DTA_EINVAL: return "invalid argument";
    case DTA_EUNSUPPORTED: return "unsupported shape (head dim must be 64 or 128)";
    case DTA_EALIGN: return "misaligned pointer";
    case DTA_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}
