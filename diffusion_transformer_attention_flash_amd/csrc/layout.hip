// Layout kernels around the local attention of context parallelism
// (diffusers "Context parallelism" guide):
// * Ulysses Attention: an all-to-all turns "all heads, my tokens" into "my
//   heads, all tokens" before the attention and back after it. Around the
//   exchange each rank splits its tensor into per-destination parts and
//   concatenates the parts it receives -- along heads on one side, along
//   tokens on the other. Ulysses Anything Attention lets both splits be
//   uneven (part sizes per rank).
// * Ring Anything Attention: ranks hold uneven token counts; the all-gather
//   moves equal-size buffers, so each part is padded to the longest before it
//   and the padding is dropped when the gathered parts are concatenated.
//
// All four operations are permutations of whole rows of D elements (one
// token of one head). One kernel covers them: each thread moves 16 bytes, a
// row is D/8 consecutive threads, and the row mapping comes from per-part
// prefix sums passed by value (P <= kMaxParts). Pure HBM-bound copies.

#include "common.h"

namespace dta {

constexpr int kMaxParts = 64;

struct PartTable {
  int64_t base[kMaxParts + 1];   // first row of part p in the packed parts buffer
  int off[kMaxParts + 1];        // prefix sum of the split axis sizes (len or heads)
  int len[kMaxParts];            // valid size along the split axis
  int pad[kMaxParts];            // stored size along the split axis (tokens only)
  int n;                         // number of parts
};

// Part p with off[p] <= x < off[p+1] (binary search; off is non-decreasing).
__device__ __forceinline__ int find_part(const PartTable& t, int64_t x, bool by_base) {
  int lo = 0, hi = t.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int64_t v = by_base ? t.base[mid] : (int64_t)t.off[mid];
    if (v <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// MODE 0 seq_concat: dst [B,H,sum len,D] <- parts [B,H,pad_p,D] (valid len_p)
// MODE 1 seq_split:  parts [B,H,pad_p,D] <- src [B,H,sum len,D], rows
//                    len_p .. pad_p-1 of each part zero-filled
// MODE 2 head_concat: dst [B,sum heads,N,D] <- parts [B,heads_p,N,D]
// MODE 3 head_split:  parts [B,heads_p,N,D] <- src [B,sum heads,N,D]
// Threads walk the destination rows; A = H (tokens modes) or N (head modes).
template <int MODE>
__global__ __launch_bounds__(256) void layout_kernel(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, PartTable t,
    int B, int A, int D, int64_t dst_rows) {
  const int cpr = D >> 3;                       // 16-byte chunks per row
  const int64_t total = dst_rows * cpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int sum_off = t.off[t.n];
  for (int64_t ci = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; ci < total;
       ci += stride) {
    const int64_t r = ci / cpr;
    const int ch = (int)(ci - r * cpr);
    int64_t sr = -1;                            // source row, -1: zero fill
    if constexpr (MODE == 0) {
      // dst row (b, h, x): x along the concatenated tokens
      const int x = (int)(r % sum_off);
      const int64_t bh = r / sum_off;
      const int p = find_part(t, x, false);
      sr = t.base[p] + bh * t.pad[p] + (x - t.off[p]);
    } else if constexpr (MODE == 1) {
      const int p = find_part(t, r, true);
      const int64_t local = r - t.base[p];
      const int xi = (int)(local % t.pad[p]);
      const int64_t bh = local / t.pad[p];
      if (xi < t.len[p]) sr = bh * sum_off + t.off[p] + xi;
    } else if constexpr (MODE == 2) {
      // dst row (b, h, n) with N = A tokens per head
      const int n = (int)(r % A);
      const int64_t bhh = r / A;
      const int h = (int)(bhh % sum_off);
      const int64_t b = bhh / sum_off;
      const int p = find_part(t, h, false);
      sr = t.base[p] + (b * t.len[p] + (h - t.off[p])) * A + n;
    } else {
      const int p = find_part(t, r, true);
      const int64_t local = r - t.base[p];
      const int n = (int)(local % A);
      const int64_t bh = local / A;
      const int hl = (int)(bh % t.len[p]);
      const int64_t b = bh / t.len[p];
      sr = (b * sum_off + t.off[p] + hl) * A + n;
    }
    u32x4 v = {0u, 0u, 0u, 0u};
    if (sr >= 0) v = *reinterpret_cast<const u32x4*>(src + sr * D + ch * 8);
    *reinterpret_cast<u32x4*>(dst + r * D + ch * 8) = v;
  }
}

}  // namespace dta

using namespace dta;

namespace {

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Validates the part sizes and fills the table. Tokens modes: sizes = len,
// padded (NULL: padded = len), rows per part = B*H*pad. Head modes: sizes =
// heads, rows per part = B*heads*N.
int make_table(PartTable& t, int P, const int* sizes, const int* padded, int64_t rows_per_unit,
               int64_t* total_units, int64_t* total_rows) {
  if (P < 1 || P > kMaxParts || !sizes) return DTA_EINVAL;
  t.n = P;
  t.off[0] = 0;
  t.base[0] = 0;
  int64_t units = 0;
  for (int p = 0; p < P; ++p) {
    const int len = sizes[p];
    const int pad = padded ? padded[p] : len;
    if (len < 0 || pad < len || pad < 1) return DTA_EINVAL;
    units += len;
    if (units > 0x7FFFFFFF) return DTA_EINVAL;
    t.len[p] = len;
    t.pad[p] = pad;
    t.off[p + 1] = (int)units;
    t.base[p + 1] = t.base[p] + rows_per_unit * pad;
  }
  if (units < 1) return DTA_EINVAL;
  *total_units = units;
  *total_rows = t.base[P];
  return DTA_OK;
}

template <int MODE>
int launch_layout(const void* src, void* dst, const PartTable& t, int B, int A, int D,
                  int64_t dst_rows, hipStream_t stream) {
  const int64_t total = dst_rows * (D / 8);
  const int64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 1 ? 1 : (want < 65536 ? want : 65536));
  hipLaunchKernelGGL(layout_kernel<MODE>, dim3(grid), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), t, B, A,
                     D, dst_rows);
  return hipGetLastError() == hipSuccess ? DTA_OK : DTA_ELAUNCH;
}

int check_common(const void* a, const void* b, int B, int X, int D) {
  if (!a || !b) return DTA_EINVAL;
  if (B < 1 || X < 1 || D < 8 || (D & 7)) return DTA_EINVAL;
  if (!al16(a) || !al16(b)) return DTA_EALIGN;
  return DTA_OK;
}

}  // namespace

extern "C" int seq_concat(const void* parts, void* out, int P, const int* lens,
                          const int* padded, int B, int H, int D, hipStream_t stream) {
  int st = check_common(parts, out, B, H, D);
  if (st != DTA_OK) return st;
  PartTable t;
  int64_t units, part_rows;
  st = make_table(t, P, lens, padded, (int64_t)B * H, &units, &part_rows);
  if (st != DTA_OK) return st;
  return launch_layout<0>(parts, out, t, B, H, D, (int64_t)B * H * units, stream);
}

extern "C" int seq_split(const void* x, void* parts, int P, const int* lens,
                         const int* padded, int B, int H, int D, hipStream_t stream) {
  int st = check_common(x, parts, B, H, D);
  if (st != DTA_OK) return st;
  PartTable t;
  int64_t units, part_rows;
  st = make_table(t, P, lens, padded, (int64_t)B * H, &units, &part_rows);
  if (st != DTA_OK) return st;
  return launch_layout<1>(x, parts, t, B, H, D, part_rows, stream);
}

extern "C" int head_concat(const void* parts, void* out, int P, const int* heads, int B,
                           int N, int D, hipStream_t stream) {
  int st = check_common(parts, out, B, N, D);
  if (st != DTA_OK) return st;
  PartTable t;
  int64_t units, part_rows;
  st = make_table(t, P, heads, nullptr, (int64_t)B * N, &units, &part_rows);
  if (st != DTA_OK) return st;
  return launch_layout<2>(parts, out, t, B, N, D, (int64_t)B * units * N, stream);
}

extern "C" int head_split(const void* x, void* parts, int P, const int* heads, int B, int N,
                          int D, hipStream_t stream) {
  int st = check_common(x, parts, B, N, D);
  if (st != DTA_OK) return st;
  PartTable t;
  int64_t units, part_rows;
  st = make_table(t, P, heads, nullptr, (int64_t)B * N, &units, &part_rows);
  if (st != DTA_OK) return st;
  return launch_layout<3>(x, parts, t, B, N, D, part_rows, stream);
}
