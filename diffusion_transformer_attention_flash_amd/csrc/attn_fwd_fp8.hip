// attn_fwd_fp8: attention on per-tensor E4M3FN Q/K/V (the fp8 dynamic
// quantisation of the ParaAttention guide, section "fp8 quantization", taken
// into the attention itself), for gfx950.
//
//   s_ij = scale * s_q * s_k * (q8_i . k8_j)             fp8 MFMA, fp32 acc
//   p_ij = exp(s_ij - m_i)       m_i = running row max of the online softmax
//   P8   = e4m3(448 * p_ij)                              P quantised to fp8
//   O_i  = s_v * sum_j P8_ij v8_j / (448 * l_i),  l_i = sum_j p_ij (fp32)
//   LSE_i = m_i + ln l_i
//
// Same structure as the bf16 kernel (S^T = K . Q^T with one query per lane,
// O^T += V^T . P^T, double-buffered K/V tiles in LDS, XCD-aware tile order),
// on v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in E4M3 and unit
// block scales: one instruction contracts 64 values. The 32 E4M3 values a
// lane supplies for P^T are its 32 exponentiated scores of the 64-key tile,
// so V^T is stored in LDS with the key bits permuted to match: the 32 keys
// of a lane half are then 32 consecutive bytes of one V^T row.

#include "common.h"

namespace dta {

template <int D, int NW>
struct Fp8Cfg {
  static constexpr int kBN = 64;
  static constexpr int kThreads = NW * 64;
  static constexpr int kBM = NW * 32;
  static constexpr int kKS = D + 16;                 // K row stride (bytes)
  static constexpr int kVS = kBN + 16;               // V^T row stride (bytes)
  static constexpr int kChunks = kBN * D / 16;       // 16-byte chunks per tile
  static constexpr int kCpt = kChunks / kThreads;
  static_assert(kChunks % kThreads == 0, "tile must split evenly");
};

// Byte position of key `key` (0..63) in a V^T row. A key 32kb + 8j + 4g + i
// (kb = bit 5, j = bits 3-4, g = bit 2, i = bits 0-1) goes to 32g + 16kb +
// 4j + i, the slot the P^T operand of lane half g holds it in.
__device__ __forceinline__ int vt8_pos(int key) {
  const int kb = (key >> 5) & 1, j = (key >> 3) & 3, g = (key >> 2) & 1, i = key & 3;
  return 32 * g + 16 * kb + 4 * j + i;
}

// Unit E8M0 block scale (2^0) for both MFMA operands.
constexpr int kUnitScale = 127;

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ v, const float* __restrict__ descale,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Nq, int Nkv,
    float scale, int n_qt) {
  using C = Fp8Cfg<D, NW>;
  constexpr int BN = C::kBN;
  __shared__ __attribute__((aligned(16))) uint8_t ks[2][BN * C::kKS];
  __shared__ __attribute__((aligned(16))) uint8_t vts[2][D * C::kVS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = blk / n_qt, qt = blk - bh * n_qt;
  const int64_t q_base = (int64_t)bh * Nq * D;
  const int64_t kv_base = (int64_t)bh * Nkv * D;
  const int row = qt * C::kBM + wave * 32 + l32;

  const float s_q = descale[0], s_k = descale[1], s_v = descale[2];
  const float c = scale * s_q * s_k * kLog2e;

  // Q^T operand: 32 bytes (dims ks*64 + 32g .. +31) per 64-dim step.
  i32x8 qr[D / 64];
#pragma unroll
  for (int kk = 0; kk < D / 64; ++kk) {
    if (row < Nq) {
      const u32x4* src = reinterpret_cast<const u32x4*>(
          q + q_base + (int64_t)row * D + kk * 64 + g * 32);
      const u32x4 lo = src[0], hi = src[1];
      qr[kk] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    } else {
      qr[kk] = i32x8{};
    }
  }

  u32x4 kreg[C::kCpt], vreg[C::kCpt];
  auto load_tile = [&](int j) {
    const int key0 = j * BN;
#pragma unroll
    for (int it = 0; it < C::kCpt; ++it) {
      const int ci = it * C::kThreads + tid;
      const int kk = ci / (D / 16), kd = ci % (D / 16);
      const int vk = ci % BN, vd = ci / BN;
      kreg[it] = (key0 + kk < Nkv)
                     ? *reinterpret_cast<const u32x4*>(
                           k + kv_base + (int64_t)(key0 + kk) * D + kd * 16)
                     : u32x4{0, 0, 0, 0};
      vreg[it] = (key0 + vk < Nkv)
                     ? *reinterpret_cast<const u32x4*>(
                           v + kv_base + (int64_t)(key0 + vk) * D + vd * 16)
                     : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < C::kCpt; ++it) {
      const int ci = it * C::kThreads + tid;
      const int kk = ci / (D / 16), kd = ci % (D / 16);
      const int vk = ci % BN, vd = ci / BN;
      *reinterpret_cast<u32x4*>(&ks[buf][kk * C::kKS + kd * 16]) = kreg[it];
      uint8_t* dst = &vts[buf][(vd * 16) * C::kVS + vt8_pos(vk)];
#pragma unroll
      for (int e = 0; e < 16; ++e)
        dst[e * C::kVS] = (uint8_t)((vreg[it][e >> 2] >> (8 * (e & 3))) & 0xFF);
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int n_tiles = (Nkv + BN - 1) / BN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const bool has_next = j + 1 < n_tiles;
    if (has_next) load_tile(j + 1);
    const uint8_t* kt = ks[buf];
    const uint8_t* vt = vts[buf];

    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4* src = reinterpret_cast<const u32x4*>(
            &kt[(kb * 32 + l32) * C::kKS + kk * 64 + g * 32]);
        const u32x4 lo = src[0], hi = src[1];
        const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a, qr[kk], s[kb], 0, 0, 0, kUnitScale, 0, kUnitScale);
      }
    }

    const bool tail = (j + 1) * BN > Nkv;
    const int key_lim = Nkv - j * BN;
    float mx = -INFINITY;
    if (tail) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= key_lim) s[kb][r] = -INFINITY;
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float rs = 0.f;
    i32x8 pb;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * w + u;
          float x = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m_new));
          if (tail) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= key_lim) x = 0.f;
          }
          rs += x;
          p[u] = x * 448.0f;
        }
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
        pb[kb * 4 + w] = wd;
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const u32x4* src = reinterpret_cast<const u32x4*>(
          &vt[(db * 32 + l32) * C::kVS + g * 32]);
      const u32x4 lo = src[0], hi = src[1];
      const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          a, pb, oacc[db], 0, 0, 0, kUnitScale, 0, kUnitScale);
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float lt = l_run + __shfl_xor(l_run, 32, 64);
  const float f = s_v / (448.0f * lt);
  if (row < Nq) {
    uint16_t* orow = o + q_base + (int64_t)row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x16& a = oacc[db];
        u32x2 w = {pack_bf16x2(a[4 * jj] * f, a[4 * jj + 1] * f),
                   pack_bf16x2(a[4 * jj + 2] * f, a[4 * jj + 3] * f)};
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * jj + 4 * g) = w;
      }
    if (g == 0 && lse != nullptr)
      lse[(int64_t)bh * Nq + row] = (m_run + log2f(lt)) * kLn2;
  }
}

template <int D, int NW>
static int launch_fp8(const void* q8, const void* k8, const void* v8,
                      const float* descale, void* o, float* lse, int B, int H,
                      int Nq, int Nkv, float scale, hipStream_t stream) {
  using C = Fp8Cfg<D, NW>;
  const int n_qt = (Nq + C::kBM - 1) / C::kBM;
  const int64_t grid = (int64_t)n_qt * B * H;
  if (grid > 0x7FFFFFFF) return DTA_EUNSUPPORTED;
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, NW>), dim3((unsigned)grid),
                     dim3(C::kThreads), 0, stream,
                     static_cast<const uint8_t*>(q8), static_cast<const uint8_t*>(k8),
                     static_cast<const uint8_t*>(v8), descale,
                     static_cast<uint16_t*>(o), lse, Nq, Nkv, scale, n_qt);
  return hipGetLastError() == hipSuccess ? DTA_OK : DTA_ELAUNCH;
}

}  // namespace dta

using namespace dta;

extern "C" int attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                            const float* descale, void* o, float* lse, int B,
                            int H, int Nq, int Nkv, int D, float scale,
                            hipStream_t stream) {
  if (!q8 || !k8 || !v8 || !descale || !o) return DTA_EINVAL;
  if (B < 1 || H < 1 || Nq < 1 || Nkv < 1) return DTA_EINVAL;
  if (!(scale >= 0.f) || !__builtin_isfinite(scale)) return DTA_EINVAL;
  if (D != 64 && D != 128) return DTA_EUNSUPPORTED;
  auto al = [](const void* p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
  };
  if (!al(q8, 16) || !al(k8, 16) || !al(v8, 16) || !al(o, 16) || !al(descale, 4) ||
      (lse && !al(lse, 4)))
    return DTA_EALIGN;
  if (D == 128)
    return launch_fp8<128, 4>(q8, k8, v8, descale, o, lse, B, H, Nq, Nkv, scale, stream);
  return launch_fp8<64, 4>(q8, k8, v8, descale, o, lse, B, H, Nq, Nkv, scale, stream);
}
