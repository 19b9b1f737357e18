// attn_merge: combine partial (O_p, LSE_p) over disjoint K/V chunks into the
// attention over their union -- the exact log-sum-exp identity that lets a
// ring-attention rank fold in each K/V block it receives (diffusers "Context
// parallelism" guide, sections "Ring Attention" and "Ring Anything
// Attention"):
//     M = max_p LSE_p, w_p = exp(LSE_p - M), W = sum_p w_p,
//     O = sum_p w_p O_p / W, LSE = M + ln W.
//
// HBM-bound scan. One thread owns 8 consecutive dims (16 bytes) of one row,
// so every load and store is a coalesced 128-bit access; the per-row LSE
// values are read by the D/8 threads of the row and served by one cache line.
// For up to 8 partials the count is a template argument and every load of a
// thread is issued before any arithmetic; more partials are visited four at
// a time. Partials are read once, with non-temporal loads, so that they
// stream past the caches instead of evicting the caller's working set.
// attn_merge_into is the two-part, in-place form used after each ring step.

#include "common.h"

namespace dta {

__device__ __forceinline__ u32x4 load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Folds partial (x, w) into the accumulator; a weight-0 partial's O is never
// used (a select, not a multiply by zero), so garbage there cannot turn into
// NaN.
__device__ __forceinline__ void merge_acc(float (&acc)[8], const u32x4& x, float w) {
  const bool live = w > 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a0 = fmaf(w, bf16_bits_to_f32(x[e] & 0xFFFF), acc[2 * e]);
    const float a1 = fmaf(w, bf16_bits_to_f32(x[e] >> 16), acc[2 * e + 1]);
    acc[2 * e] = live ? a0 : acc[2 * e];
    acc[2 * e + 1] = live ? a1 : acc[2 * e + 1];
  }
}

__device__ __forceinline__ void merge_store(uint16_t* o, float* lse, int64_t row, int ch, int D,
                                            float (&acc)[8], float m, float wsum) {
  if (m != -INFINITY) {
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
  }
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
  *reinterpret_cast<u32x4*>(o + row * D + ch * 8) = out;
  if (ch == 0 && lse != nullptr) lse[row] = (m == -INFINITY) ? -INFINITY : m + logf(wsum);
}

// N partials (1..8): all loads of the thread first, then the arithmetic.
template <int D, int N>
__global__ __launch_bounds__(256) void attn_merge_n_kernel(
    const uint16_t* __restrict__ op, const float* __restrict__ lp,
    uint16_t* __restrict__ o, float* __restrict__ lse, int64_t rows) {
  constexpr int kCh = D / 8;
  const int64_t total = rows * kCh;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t ci = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; ci < total;
       ci += stride) {
    const int64_t row = ci / kCh;
    const int ch = (int)(ci - row * kCh);
    u32x4 x[N];
    float l[N];
#pragma unroll
    for (int p = 0; p < N; ++p) {
      x[p] = load_stream(op + ((int64_t)p * rows + row) * D + ch * 8);
      l[p] = lp[(int64_t)p * rows + row];
    }
    float m = -INFINITY;
#pragma unroll
    for (int p = 0; p < N; ++p) m = fmaxf(m, l[p]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (m != -INFINITY) {
      const float ml2 = m * kLog2e;
#pragma unroll
      for (int p = 0; p < N; ++p) {
        const float w = __builtin_amdgcn_exp2f(fmaf(l[p], kLog2e, -ml2));
        wsum += w;
        merge_acc(acc, x[p], w);
      }
    }
    merge_store(o, lse, row, ch, D, acc, m, wsum);
  }
}

// Any number of partials, four at a time.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const uint16_t* __restrict__ op, const float* __restrict__ lp, int n,
    uint16_t* __restrict__ o, float* __restrict__ lse, int64_t rows) {
  constexpr int kCh = D / 8;
  const int64_t total = rows * kCh;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t ci = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; ci < total;
       ci += stride) {
    const int64_t row = ci / kCh;
    const int ch = (int)(ci - row * kCh);
    float m = -INFINITY;
    for (int p = 0; p < n; ++p) m = fmaxf(m, lp[(int64_t)p * rows + row]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (m != -INFINITY) {
      const float ml2 = m * kLog2e;
      int p = 0;
      for (; p + 4 <= n; p += 4) {
        u32x4 x[4];
        float w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          x[u] = load_stream(op + ((int64_t)(p + u) * rows + row) * D + ch * 8);
          w[u] = __builtin_amdgcn_exp2f(
              fmaf(lp[(int64_t)(p + u) * rows + row], kLog2e, -ml2));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          wsum += w[u];
          merge_acc(acc, x[u], w[u]);
        }
      }
      for (; p < n; ++p) {
        const u32x4 x = load_stream(op + ((int64_t)p * rows + row) * D + ch * 8);
        const float w = __builtin_amdgcn_exp2f(
            fmaf(lp[(int64_t)p * rows + row], kLog2e, -ml2));
        wsum += w;
        merge_acc(acc, x, w);
      }
    }
    merge_store(o, lse, row, ch, D, acc, m, wsum);
  }
}

// (o, lse) <- merge((o, lse), (op, lp)), in place. The D/8 threads of a row
// are consecutive lanes of one wave, so every lane of the row reads lse[row]
// before the row's first lane overwrites it.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_into_kernel(
    uint16_t* __restrict__ o, float* __restrict__ lse, const uint16_t* __restrict__ op,
    const float* __restrict__ lp, int64_t rows) {
  constexpr int kCh = D / 8;
  static_assert(64 % kCh == 0, "a row must not straddle two waves");
  const int64_t total = rows * kCh;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t ci = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; ci < total;
       ci += stride) {
    const int64_t row = ci / kCh;
    const int ch = (int)(ci - row * kCh);
    const float la = lse[row], lb = lp[row];
    const u32x4 xa = *reinterpret_cast<const u32x4*>(o + row * D + ch * 8);
    const u32x4 xb = *reinterpret_cast<const u32x4*>(op + row * D + ch * 8);
    const float m = fmaxf(la, lb);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float lout = -INFINITY;
    if (m != -INFINITY) {
      const float ml2 = m * kLog2e;
      const float wa = __builtin_amdgcn_exp2f(fmaf(la, kLog2e, -ml2));
      const float wb = __builtin_amdgcn_exp2f(fmaf(lb, kLog2e, -ml2));
      const float inv = 1.0f / (wa + wb);
      const float fa = wa * inv, fb = wb * inv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // A part of weight 0 contributes nothing, whatever its O holds.
        const float a0 = bf16_bits_to_f32(xa[e] & 0xFFFF), a1 = bf16_bits_to_f32(xa[e] >> 16);
        const float b0 = bf16_bits_to_f32(xb[e] & 0xFFFF), b1 = bf16_bits_to_f32(xb[e] >> 16);
        acc[2 * e] = (wa > 0.f ? fa * a0 : 0.f) + (wb > 0.f ? fb * b0 : 0.f);
        acc[2 * e + 1] = (wa > 0.f ? fa * a1 : 0.f) + (wb > 0.f ? fb * b1 : 0.f);
      }
      lout = m + logf(wa + wb);
    }
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
    *reinterpret_cast<u32x4*>(o + row * D + ch * 8) = out;
    if (ch == 0) lse[row] = lout;
  }
}

template <int D>
void launch_merge(const void* o_parts, const float* lse_parts, int n, void* o, float* lse,
                  int64_t rows, unsigned grid, hipStream_t stream) {
  const uint16_t* op = static_cast<const uint16_t*>(o_parts);
  uint16_t* out = static_cast<uint16_t*>(o);
  switch (n) {
#define DTA_MERGE_N(N)                                                                       \
  case N:                                                                                    \
    hipLaunchKernelGGL((attn_merge_n_kernel<D, N>), dim3(grid), dim3(256), 0, stream, op,    \
                       lse_parts, out, lse, rows);                                           \
    break;
    DTA_MERGE_N(1)
    DTA_MERGE_N(2)
    DTA_MERGE_N(3)
    DTA_MERGE_N(4)
    DTA_MERGE_N(5)
    DTA_MERGE_N(6)
    DTA_MERGE_N(7)
    DTA_MERGE_N(8)
#undef DTA_MERGE_N
    default:
      hipLaunchKernelGGL(attn_merge_kernel<D>, dim3(grid), dim3(256), 0, stream, op, lse_parts,
                         n, out, lse, rows);
  }
}

}  // namespace dta

using namespace dta;

extern "C" int attn_merge(const void* o_parts, const float* lse_parts,
                          int n_parts, void* o, float* lse, int B, int H,
                          int Nq, int D, hipStream_t stream) {
  if (!o_parts || !lse_parts || !o) return DTA_EINVAL;
  if (n_parts < 1 || B < 1 || H < 1 || Nq < 1) return DTA_EINVAL;
  if (D != 64 && D != 128) return DTA_EUNSUPPORTED;
  auto al = [](const void* p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
  };
  if (!al(o_parts, 16) || !al(o, 16) || !al(lse_parts, 4) || (lse && !al(lse, 4)))
    return DTA_EALIGN;
  const int64_t rows = (int64_t)B * H * Nq;
  const int64_t total = rows * (D / 8);
  const int64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  if (D == 128)
    launch_merge<128>(o_parts, lse_parts, n_parts, o, lse, rows, grid, stream);
  else
    launch_merge<64>(o_parts, lse_parts, n_parts, o, lse, rows, grid, stream);
  return hipGetLastError() == hipSuccess ? DTA_OK : DTA_ELAUNCH;
}

extern "C" int attn_merge_into(void* o, float* lse, const void* o_part,
                               const float* lse_part, int B, int H, int Nq, int D,
                               hipStream_t stream) {
  if (!o || !lse || !o_part || !lse_part) return DTA_EINVAL;
  if (B < 1 || H < 1 || Nq < 1) return DTA_EINVAL;
  if (D != 64 && D != 128) return DTA_EUNSUPPORTED;
  auto al = [](const void* p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
  };
  if (!al(o, 16) || !al(o_part, 16) || !al(lse, 4) || !al(lse_part, 4)) return DTA_EALIGN;
  const int64_t rows = (int64_t)B * H * Nq;
  const int64_t total = rows * (D / 8);
  const int64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  if (D == 128)
    hipLaunchKernelGGL(attn_merge_into_kernel<128>, dim3(grid), dim3(256), 0, stream,
                       static_cast<uint16_t*>(o), lse, static_cast<const uint16_t*>(o_part),
                       lse_part, rows);
  else
    hipLaunchKernelGGL(attn_merge_into_kernel<64>, dim3(grid), dim3(256), 0, stream,
                       static_cast<uint16_t*>(o), lse, static_cast<const uint16_t*>(o_part),
                       lse_part, rows);
  return hipGetLastError() == hipSuccess ? DTA_OK : DTA_ELAUNCH;
}
