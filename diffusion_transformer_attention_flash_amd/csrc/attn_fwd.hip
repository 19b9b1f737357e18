// attn_fwd: non-causal multi-head attention forward, bf16 in, bf16 O and
// float32 natural-log LSE out, for gfx950 (CDNA4).
//
// Operation: O_i = sum_j exp(s_ij) v_j / sum_j exp(s_ij), s_ij = scale q_i.k_j,
// LSE_i = ln sum_j exp(s_ij) -- the attention every SDPA backend computes
// (diffusers "Accelerate inference" guide, section "Scaled dot product
// attention"), evaluated by tiles with an online softmax, which rearranges
// the same sums exactly.
//
// Design (one workgroup = NW waves = NW*QB*32 query rows of one (b, h)):
// * The scores are computed transposed, S^T = K . Q^T, on
//   v_mfma_f32_32x32x16_bf16: K rows come from LDS as the A operand and the
//   wave's Q rows sit in registers as the B operand for the whole K/V loop.
//   In the 32x32 accumulator layout lane l then owns query l%32 and 16 of the
//   32 keys (rows 8*(r/4) + 4*(l/32) + r%4 of register r), so the row max and
//   row sum need only in-lane work plus one exchange between the two wave
//   halves.
// * O is accumulated transposed too, O^T += V^T . P^T: the exponentiated
//   scores, rounded to bf16, are the B operand straight from the registers
//   that held S^T, and V^T comes from LDS. The contraction over keys only
//   needs A and B to enumerate the same keys in the same (lane half, item)
//   slots, so V^T is written to LDS with bits 2 and 3 of the key index
//   swapped: the 8 keys a lane's P operand holds are then 8 consecutive
//   bf16 of one V^T row (one 128-bit LDS read).
// * K/V tiles (BN keys) are double-buffered in LDS; the next tile's global
//   loads are issued before the current tile's MFMAs and land in the other
//   buffer afterwards, so one barrier per tile suffices.
// * Softmax runs in the log2 domain: c = scale*log2(e) is folded into one FMA
//   per score before v_exp_f32. Only the last, partial tile masks keys.
// * Workgroup ids are remapped so that the workgroups of one XCD walk
//   consecutive query tiles of the same head and share K/V through its L2.

#include "common.h"

namespace dta {

template <int D, int NW, int QB, int BN>
struct AttnCfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kBM = NW * QB * 32;          // query rows per workgroup
  static constexpr int kKS = D + 8;                 // K tile row stride (elements)
  static constexpr int kVS = BN + 8;                // V^T tile row stride (elements)
  static constexpr int kKElems = BN * kKS;
  static constexpr int kVElems = D * kVS;
  static constexpr int kChunks = BN * D / 8;        // 16-byte chunks per tile
  static constexpr int kCpt = kChunks / kThreads;   // chunks per thread
  static_assert(kChunks % kThreads == 0, "tile must split evenly");
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
};

// Position of key `key` (0..BN-1) inside a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~0xC) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <int D, int NW, int QB, int BN>
__global__ __launch_bounds__(NW * 64) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int Nq, int Nkv, float c, int n_qt) {
  using C = AttnCfg<D, NW, QB, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][C::kKElems];
  __shared__ __attribute__((aligned(16))) uint16_t vts[2][C::kVElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = blk / n_qt, qt = blk - bh * n_qt;
  const int64_t q_base = (int64_t)bh * Nq * D;
  const int64_t kv_base = (int64_t)bh * Nkv * D;
  const int q0 = qt * C::kBM + wave * QB * 32;

  // Q^T operand: query q0 + qb*32 + l32, dims ds*16 + 8g .. +7.
  bf16x8 qr[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = q0 + qb * 32 + l32;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      if (row < Nq) {
        qr[qb][ds] = *reinterpret_cast<const bf16x8*>(
            q + q_base + (int64_t)row * D + ds * 16 + g * 8);
      } else {
        qr[qb][ds] = bf16x8{};
      }
    }
  }

  // K tile chunk mapping: 16 consecutive threads read one key row (coalesced).
  // V tile chunk mapping: consecutive threads read consecutive keys, so the
  // transposed 16-bit LDS writes of one wave fill one V^T row.
  u32x4 kreg[C::kCpt], vreg[C::kCpt];
  auto load_tile = [&](int j) {
    const int key0 = j * BN;
#pragma unroll
    for (int it = 0; it < C::kCpt; ++it) {
      const int ci = it * C::kThreads + tid;
      const int kk = ci / (D / 8), kd = ci % (D / 8);
      const int vk = ci % BN, vd = ci / BN;
      kreg[it] = (key0 + kk < Nkv)
                     ? *reinterpret_cast<const u32x4*>(
                           k + kv_base + (int64_t)(key0 + kk) * D + kd * 8)
                     : u32x4{0, 0, 0, 0};
      vreg[it] = (key0 + vk < Nkv)
                     ? *reinterpret_cast<const u32x4*>(
                           v + kv_base + (int64_t)(key0 + vk) * D + vd * 8)
                     : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < C::kCpt; ++it) {
      const int ci = it * C::kThreads + tid;
      const int kk = ci / (D / 8), kd = ci % (D / 8);
      const int vk = ci % BN, vd = ci / BN;
      *reinterpret_cast<u32x4*>(&ks[buf][kk * C::kKS + kd * 8]) = kreg[it];
      uint16_t* dst = &vts[buf][(vd * 8) * C::kVS + vt_pos(vk)];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[(2 * e) * C::kVS] = (uint16_t)(vreg[it][e] & 0xFFFF);
        dst[(2 * e + 1) * C::kVS] = (uint16_t)(vreg[it][e] >> 16);
      }
    }
  };

  f32x16 oacc[QB][D / 32];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[qb][db] = f32x16{};
  }

  const int n_tiles = (Nkv + BN - 1) / BN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const bool has_next = j + 1 < n_tiles;
    if (has_next) load_tile(j + 1);
    const uint16_t* kt = ks[buf];
    const uint16_t* vt = vts[buf];

    // S^T = K . Q^T for BN keys x 32 queries per query block.
    f32x16 s[QB][BN / 32];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &kt[(kb * 32 + l32) * C::kKS + ds * 16 + g * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a, qr[qb][ds], s[qb][kb], 0, 0, 0);
      }
    }

    // Online softmax (log2 domain). Keys past Nkv exist only in the last tile.
    const bool tail = (j + 1) * BN > Nkv;
    const int key_lim = Nkv - j * BN;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
      if (tail) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= key_lim) s[qb][kb][r] = -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[qb], mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r], c, -m_new));
          if (tail) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= key_lim) p = 0.f;
          }
          s[qb][kb][r] = p;
          rs += p;
        }
      l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[qb][db] *= alpha;
    }

    // O^T += V^T . P^T, 16 keys per MFMA.
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 pb[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const f32x16& sv = s[qb][kb];
          pb[qb] = bf16x8{(__bf16)sv[8 * t + 0], (__bf16)sv[8 * t + 1],
                          (__bf16)sv[8 * t + 2], (__bf16)sv[8 * t + 3],
                          (__bf16)sv[8 * t + 4], (__bf16)sv[8 * t + 5],
                          (__bf16)sv[8 * t + 6], (__bf16)sv[8 * t + 7]};
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              &vt[(db * 32 + l32) * C::kVS + kb * 32 + 16 * t + 8 * g]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a, pb[qb], oacc[qb][db], 0, 0, 0);
        }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane owns query row (l32) and dims db*32 + 8*(r/4) + 4g + r%4.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    const float inv = 1.0f / lt;
    const int row = q0 + qb * 32 + l32;
    if (row < Nq) {
      uint16_t* orow = o + q_base + (int64_t)row * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x16& a = oacc[qb][db];
          u32x2 w = {pack_bf16x2(a[4 * jj] * inv, a[4 * jj + 1] * inv),
                     pack_bf16x2(a[4 * jj + 2] * inv, a[4 * jj + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * jj + 4 * g) = w;
        }
      if (g == 0 && lse != nullptr)
        lse[(int64_t)bh * Nq + row] = (m_run[qb] + log2f(lt)) * kLn2;
    }
  }
}

template <int D, int NW, int QB, int BN>
static int launch_attn_fwd(const void* q, const void* k, const void* v,
                           void* o, float* lse, int B, int H, int Nq, int Nkv,
                           float scale, hipStream_t stream) {
  using C = AttnCfg<D, NW, QB, BN>;
  const int n_qt = (Nq + C::kBM - 1) / C::kBM;
  const int64_t grid = (int64_t)n_qt * B * H;
  if (grid > 0x7FFFFFFF) return DTA_EUNSUPPORTED;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW, QB, BN>), dim3((unsigned)grid),
                     dim3(C::kThreads), 0, stream,
                     static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o),
                     lse, Nq, Nkv, scale * kLog2e, n_qt);
  return hipGetLastError() == hipSuccess ? DTA_OK : DTA_ELAUNCH;
}

}  // namespace dta

using namespace dta;

static bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o,
                        float* lse, int B, int H, int Nq, int Nkv, int D,
                        float scale, hipStream_t stream) {
  if (!q || !k || !v || !o) return DTA_EINVAL;
  if (B < 1 || H < 1 || Nq < 1 || Nkv < 1) return DTA_EINVAL;
  if (!(scale >= 0.f) || !__builtin_isfinite(scale)) return DTA_EINVAL;
  if (D != 64 && D != 128) return DTA_EUNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return DTA_EALIGN;
  if (D == 128)
    return launch_attn_fwd<128, 4, 1, 64>(q, k, v, o, lse, B, H, Nq, Nkv, scale, stream);
  return launch_attn_fwd<64, 4, 1, 64>(q, k, v, o, lse, B, H, Nq, Nkv, scale, stream);
}
