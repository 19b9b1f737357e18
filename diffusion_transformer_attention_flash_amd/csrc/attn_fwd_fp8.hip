// attn_fwd_fp8: attention on per-tensor E4M3FN Q/K/V (the fp8 dynamic
// quantisation of the ParaAttention guide, section "fp8 quantization", taken
// into the attention itself), for gfx950.
//
//   s_ij = scale * s_q * s_k * (q8_i . k8_j)             fp8 MFMA, fp32 acc
//   p_ij = exp(s_ij - m_i)   m_i = the online softmax's reference max, which
//                            trails the running row max by at most 2 bits:
//                            p_ij <= 4
//   P8   = e4m3(108 * p_ij)                 P quantised to fp8, <= 432
//   O_i  = s_v * sum_j P8_ij v8_j / (108 * l_i),  l_i = sum_j p_ij (fp32)
//   LSE_i = m_i + ln l_i
//
// Same structure as the bf16 kernel: S^T = K . Q^T with one query per lane,
// O^T += V^T . P^T, padded K/V tiles in LDS fed by buffer loads whose range
// check zero-fills rows past Nkv, a peeled masked tail tile, a reference max
// raised only when a row outgrows it, XCD-aware tile order.
// * At D = 128 with per-tensor or per-token Q/K scales a workgroup is 8 waves
//   (two per SIMD) and the waves of the second half run skewed: each tile
//   they first finish the previous tile's P.V, then score the current one, so
//   the softmax of one wave of a SIMD falls under the other's MFMAs instead of
//   beside them (the fp8 MFMA leaves about as much VALU work as MFMA work per
//   tile). P.V one tile late needs that tile's V for one more barrier
//   interval: three LDS buffers, still one barrier per tile. The other
//   instances are 4 waves with two buffers. The 8-wave instances also stage
//   O through LDS in the epilogue, so that each global store covers whole
//   output rows.
// The MFMA is v_mfma_f32_32x32x64_f8f6f4 with both operands E4M3: one
// instruction contracts 64 values, so a 64-key tile takes one P.V MFMA per 32
// head dims.
// * 108 p is produced directly as exp2(c s - (m - log2 108)), so quantising
//   P costs only the packed conversion; the row sum of these values is
//   108 l. The 2-bit slack of the reference max keeps the O rescale rare
//   while 108 p stays inside the E4M3 range with a 3.7% margin for the
//   rounding of v_exp_f32 (the largest finite E4M3 value is 448).
// * The P^T operand of lane half g is its 32 scores of the tile in register
//   order, i.e. keys 32(i/16) + 8((i%16)/4) + 4g + i%4 for byte i. The V tile
//   is written to LDS with its key index permuted (key bit 2 -> row bit 5,
//   key bits 3-5 -> row bits 2-4), so those 32 keys are rows 32g .. 32g+31,
//   and four ds_read_b64_tr_b8 -- each handing a lane one head dimension of
//   8 consecutive rows -- assemble the V^T operand in the same byte order.

#include <type_traits>

#include "common.h"

namespace dta {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <int D, int NW>
struct Fp8Cfg {
  static constexpr int kBN = 64;
  static constexpr int kThreads = NW * 64;
  static constexpr int kBM = NW * 32;
  static constexpr int kKS = D + 16;                 // K row stride (bytes)
  static constexpr int kVS = D + 32;                 // V row stride (bytes)
  static constexpr int kCPR = D / 16;                // 16-byte chunks per row
  static constexpr int kChunks = kBN * kCPR;
  static constexpr int kCpt = kChunks / kThreads;
  static_assert(kChunks % kThreads == 0, "tile must split evenly");
};

constexpr float kTau8 = 2.0f;                    // reference-max slack (log2)
constexpr float kLog2PScale = 6.754887502163468f; // log2(108): 108 * 2^kTau8 <= 448
constexpr int kBufDword3Fp8 = 0x00020000;

// LDS row of key `key` (0..63) in the V tile.
__device__ __forceinline__ int v8_row(int key) {
  return (((key >> 2) & 1) << 5) | (((key >> 3) & 7) << 2) | (key & 3);
}

__device__ __forceinline__ float xhalf_max8(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum8(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// MODE 0: per-tensor scales descale[0..2] for Q, K, V.
// MODE 1 (rows): Q and K carry one power-of-two scale per token (E8M0 bytes
// q_e8, k_e8); the score MFMA applies them through its operand scales (A row
// = key, B column = query), and descale[0] is V's per-tensor scale.
// MODE 2 (rows_v): as MODE 1, and V carries one power-of-two scale per token
// (E8M0 bytes v_e8). V's scale is folded into the probabilities,
// pv = p * 2^(ev - 127), which are quantised with one power-of-two scale per
// (query, block of 32 consecutive keys). The fp8 MFMA applies one operand
// scale to each 32 consecutive k of a column, taken from lane half
// kb of that column (measured: bytes 0-15 of every lane are scaled by the
// lower lanes' scale, bytes 16-31 by the upper lanes'), and a lane's P bytes
// 0-15 / 16-31 are its keys of block kb = 0 / 1. So each block's max is
// reduced over the lane pair (l, l ^ 32) and lane half g supplies block g's
// scale to the P.V MFMA.
template <int D, int NW, int MODE>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ v, const float* __restrict__ descale,
    const uint8_t* __restrict__ q_e8, const uint8_t* __restrict__ k_e8,
    const uint8_t* __restrict__ v_e8, uint16_t* __restrict__ o, float* __restrict__ lse,
    int Nq, int Nkv, float scale, int n_qt) {
  constexpr bool ROWS = MODE >= 1;
  using C = Fp8Cfg<D, NW>;
  constexpr int BN = C::kBN;
  constexpr bool SKEW = NW == 8;
  constexpr int NBUF = SKEW ? 3 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t ks[NBUF][BN * C::kKS];
  __shared__ __attribute__((aligned(16))) uint8_t vs[NBUF][BN * C::kVS];
  // MODE 2: the V scales 2^(e - 127) of the tile's keys, as floats.
  __shared__ __attribute__((aligned(16))) float ves[NBUF][MODE == 2 ? BN : 4];
  // Epilogue staging of O (the 8-wave instances): 32 rows of 272 bytes per
  // wave. (The 4-wave rows_v instance keeps direct stores: two workgroups
  // share a CU there, and its video-shape time rose 0.7% with the staging.)
  __shared__ __attribute__((aligned(16))) uint8_t ostg[NW == 8 ? NW * 32 * 272 : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const bool late = SKEW && __builtin_amdgcn_readfirstlane(wave) >= NW / 2;
  const int g = lane >> 5, l32 = lane & 31;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = blk / n_qt, qt = blk - bh * n_qt;
  const int64_t q_base = (int64_t)bh * Nq * D;
  const uint8_t* kh = k + (int64_t)bh * Nkv * D;
  const uint8_t* vh = v + (int64_t)bh * Nkv * D;
  const int row = qt * C::kBM + wave * 32 + l32;

  const float s_q = ROWS ? 1.0f : descale[0], s_k = ROWS ? 1.0f : descale[1];
  const float s_v = MODE == 2 ? 1.0f : (ROWS ? descale[0] : descale[2]);
  const float c = scale * s_q * s_k * kLog2e;
  // E8M0 operand scales of the score MFMA (127 = 2^0).
  const int sq_e = (ROWS && row < Nq) ? (int)q_e8[(int64_t)bh * Nq + row] : 127;
  const uint8_t* ke_h = ROWS ? k_e8 + (int64_t)bh * Nkv : nullptr;
  const uint8_t* ve_h = MODE == 2 ? v_e8 + (int64_t)bh * Nkv : nullptr;
  int sk_next[2] = {127, 127};
  int ve_next = 127;                     // V exponent byte of key tid (tid < BN)

  // Q^T operand: 32 bytes (dims kk*64 + 32g .. +31) per 64-dim step.
  i32x8 qr[D / 64];
#pragma unroll
  for (int kk = 0; kk < D / 64; ++kk) {
    if (row < Nq) {
      const u32x4* src = reinterpret_cast<const u32x4*>(
          q + q_base + (int64_t)row * D + kk * 64 + g * 32);
      qr[kk] = cat8(src[0], src[1]);
    } else {
      qr[kk] = i32x8{};
    }
  }

  // Staging: chunk ci -> key ci / kCPR, 16-byte chunk ci % kCPR.
  const int st_r = tid / C::kCPR, st_c = tid % C::kCPR;
  constexpr int kRowsPerIt = C::kThreads / C::kCPR;
  u32x4 kreg[C::kCpt], vreg[C::kCpt];
  auto load_tile = [&](int j) {
    const int64_t key0 = (int64_t)j * BN;
    const int bytes = (int)min<int64_t>((int64_t)(Nkv - key0) * D, (int64_t)BN * D);
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kh + key0 * D), 0, bytes, kBufDword3Fp8);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vh + key0 * D), 0, bytes, kBufDword3Fp8);
#pragma unroll
    for (int it = 0; it < C::kCpt; ++it) {
      const int off = (st_r + it * kRowsPerIt) * D + st_c * 16;
      kreg[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0);
      vreg[it] = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
    }
    if constexpr (ROWS) {
      // Scales of the keys this lane's A rows hold. Keys past Nkv read the
      // last key's scale (clamped address, no branch): their K rows are zero
      // and their scores are masked, so the value is never used.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int64_t key = min<int64_t>(key0 + kb * 32 + l32, (int64_t)Nkv - 1);
        sk_next[kb] = (int)ke_h[key];
      }
    }
    if constexpr (MODE == 2) {
      // Same clamp: a key past Nkv has a zero V row and zero probability.
      if (tid < BN) ve_next = (int)ve_h[min<int64_t>(key0 + tid, (int64_t)Nkv - 1)];
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < C::kCpt; ++it) {
      const int r = st_r + it * kRowsPerIt;
      *reinterpret_cast<u32x4*>(&ks[buf][r * C::kKS + st_c * 16]) = kreg[it];
      *reinterpret_cast<u32x4*>(&vs[buf][v8_row(r) * C::kVS + st_c * 16]) = vreg[it];
    }
    if constexpr (MODE == 2) {
      if (tid < BN) ves[buf][tid] = __builtin_amdgcn_ldexpf(1.0f, ve_next - 127);
    }
  };

  // Operand read bases: K rows l32 (A operand), V^T rows 32g + 8a + s/2 at
  // byte 16*(lane/16 % 2) + 8*(s%2) of a 32-dim block, s = lane % 16.
  const int k_base = l32 * C::kKS + g * 32;
  const int v_base = (32 * g + ((lane & 15) >> 1)) * C::kVS + 16 * ((lane >> 4) & 1) +
                     8 * (lane & 1);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int n_tiles = (Nkv + BN - 1) / BN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  // S^T of tile j (K in kt, V scales in vte_buf for MODE 2) and its
  // softmax into the P operand pb and its scale sb_e.
  auto qk_softmax = [&](int j, const uint8_t* kt, const float* vte_buf, const int (&sk_e)[2],
                        i32x8& pb, int& sb_e, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4* src = reinterpret_cast<const u32x4*>(kt + k_base + kb * 32 * C::kKS + kk * 64);
        if constexpr (ROWS)
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              cat8(src[0], src[1]), qr[kk], s[kb], 0, 0, 0, sk_e[kb], 0, sq_e);
        else
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              cat8(src[0], src[1]), qr[kk], s[kb], 0, 0, 0, 0, 0, 0);
      }

    const int key_lim = Nkv - j * BN;
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3) >= key_lim) s[kb][r] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = xhalf_max8(mx) * c;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kTau8) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    sb_e = 127;
    if constexpr (MODE != 2) {
      const float m448 = m_run - kLog2PScale;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float p[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * w + u;
            p[u] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m448));
            if constexpr (MASK) {
              if (kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3) >= key_lim) p[u] = 0.f;
            }
            rs += p[u];
          }
          // The first conversion writes the low half; the high half of `old`
          // (any dead register, here p[0]'s) is overwritten by the second.
          int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);
          wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
          pb[kb * 4 + w] = wd;
          asm volatile("" : "+v"(rs));
        }
      l_run += rs;
    } else {
      // p = 2^(s c - m_run) in (0, 2^kTau8]; l_run sums p. pv = p 2^(ev-127)
      // for this lane's keys kb*32 + 8w + 4g + u (4 consecutive V scales per
      // (kb, w): one aligned 16-byte LDS read).
      const float* vte = vte_buf;
      float pv[2][16];
      float rs = 0.f, bmax[2] = {0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x4 ev = *reinterpret_cast<const f32x4*>(vte + kb * 32 + 8 * w + 4 * g);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * w + u;
            float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m_run));
            if constexpr (MASK) {
              if (kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3) >= key_lim) p = 0.f;
            }
            rs += p;
            pv[kb][r] = p * ev[u];        // exact: a power-of-two factor
            bmax[kb] = fmaxf(bmax[kb], pv[kb][r]);
          }
          asm volatile("" : "+v"(rs));
        }
      l_run += rs;
      // Block exponent: the smallest e with bmax <= 448 * 2^e, read off the
      // float32 bits of bmax = (1 + f/2^23) 2^(E-127): 448 * 2^e = 1.75 *
      // 2^(8+e), so e = E - 135 when 1 + f/2^23 <= 1.75, else E - 134.
      // Clamped to [-126, 127] (a block below 448 * 2^-127 still fits
      // 2^-126 exactly, and keeps the conversion scale a normal float).
      int ebk[2];
      float sck[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float bm = xhalf_max8(bmax[kb]);          // the block's 32 keys
        const uint32_t bb = __float_as_uint(bm);
        const int E = (int)(bb >> 23);
        int eb = (bb & 0x7FFFFFu) <= 0x600000u ? E - 135 : E - 134;
        eb = bm > 0.f ? max(min(eb, 127), -126) : 0;
        ebk[kb] = eb;
        sck[kb] = __builtin_amdgcn_ldexpf(1.0f, eb);
      }
      sb_e = (g == 0 ? ebk[0] : ebk[1]) + 127;
      typedef short s16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // pv / 2^eb <= 448: the unsaturated scaled conversion cannot overflow.
          s16x2 wd = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
              s16x2{0, 0}, pv[kb][4 * w], pv[kb][4 * w + 1], sck[kb], false);
          wd = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(wd, pv[kb][4 * w + 2], pv[kb][4 * w + 3],
                                                        sck[kb], true);
          pb[kb * 4 + w] = __builtin_bit_cast(int, wd);
        }
    }
  };
  // O^T += V^T . P^T for the tile whose V is in vt.
  auto pv = [&](const uint8_t* vt, const i32x8& pb, int sb_e) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      i32x2 part[4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        part[a] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2*)(vt + v_base + 8 * a * C::kVS + db * 32));
      const i32x8 av = {part[0][0], part[0][1], part[1][0], part[1][1],
                        part[2][0], part[2][1], part[3][0], part[3][1]};
      if constexpr (MODE == 2)
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb, oacc[db], 0, 0, 0,
                                                                    127, 0, sb_e);
      else
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb, oacc[db], 0, 0, 0, 0,
                                                                    0, 0);
    }
  };
  i32x8 pb_late = {};
  int sb_late = 127;
  // One K/V tile in buffer buf = j % NBUF; MASK only for a ragged last tile.
  // The late waves (the second wave of every SIMD) finish tile j-1 first (its
  // P is in pb_late, its V still in buffer (j-1) % NBUF), then score tile j;
  // their last P.V follows the loop. The tile staged during tile j goes to
  // buffer (j+1) % NBUF, which no wave reads in this barrier interval.
  auto tile = [&](int j, auto buf_tag, auto mask_tag,
                  auto late_tag) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_tag)::value;
    constexpr bool LATE = decltype(late_tag)::value;
    constexpr int pbuf = (buf + NBUF - 1) % NBUF;
    const bool has_next = j + 1 < n_tiles;
    const int sk_e[2] = {sk_next[0], sk_next[1]};
    if (has_next) load_tile(j + 1);
    if constexpr (LATE) {
      if (j > 0) pv(vs[pbuf], pb_late, sb_late);
      qk_softmax(j, ks[buf], ves[buf], sk_e, pb_late, sb_late, mask_tag);
    } else {
      i32x8 pb;
      int sb_e;
      qk_softmax(j, ks[buf], ves[buf], sk_e, pb, sb_e, mask_tag);
      pv(vs[buf], pb, sb_e);
    }
    debug_sync();
    if (has_next) store_tile((buf + 1) % NBUF);
    __syncthreads();
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  const int n_full = (Nkv % BN == 0) ? n_tiles : n_tiles - 1;
  auto run = [&](auto late_tag) __attribute__((always_inline)) {
    constexpr bool LATE = decltype(late_tag)::value;
    int j = 0;
    if constexpr (NBUF == 3) {
      for (; j + 2 < n_full; j += 3) {
        tile(j, B0{}, std::false_type{}, late_tag);
        tile(j + 1, B1{}, std::false_type{}, late_tag);
        tile(j + 2, B2{}, std::false_type{}, late_tag);
      }
      for (; j < n_full; ++j) {
        if (j % 3 == 0)
          tile(j, B0{}, std::false_type{}, late_tag);
        else
          tile(j, B1{}, std::false_type{}, late_tag);
      }
      if (j < n_tiles) {
        if (j % 3 == 0)
          tile(j, B0{}, std::true_type{}, late_tag);
        else if (j % 3 == 1)
          tile(j, B1{}, std::true_type{}, late_tag);
        else
          tile(j, B2{}, std::true_type{}, late_tag);
      }
      if constexpr (LATE) {
        const int lb = (n_tiles - 1) % 3;
        pv(vs[lb], pb_late, sb_late);
      }
    } else {
      for (; j + 1 < n_full; j += 2) {
        tile(j, B0{}, std::false_type{}, late_tag);
        tile(j + 1, B1{}, std::false_type{}, late_tag);
      }
      if (j < n_full) tile(j++, B0{}, std::false_type{}, late_tag);
      if (j < n_tiles) {
        if (j & 1)
          tile(j, B1{}, std::true_type{}, late_tag);
        else
          tile(j, B0{}, std::true_type{}, late_tag);
      }
    }
  };
  if (late)
    run(std::true_type{});
  else
    run(std::false_type{});

  debug_sync();
  // MODE 0/1: l_run holds 108 l and O = s_v * acc / (108 l). MODE 2: l_run
  // holds l and O = acc / l (V's scale is in P).
  const float lt = xhalf_sum8(l_run);
  const float f = s_v / lt;
  if constexpr (D == 128 && NW == 8) {
    // O goes through LDS so that each global store covers whole 256-byte
    // rows (16 lanes per row) instead of 16 bytes of each of 32 rows. Each
    // wave stages its 32 rows (272-byte pitch) in its own slice and reads
    // back only that slice: no barrier. Every lane takes part, since the rows
    // a lane stores are not its own; the indices derive from `row` and `g`.
    constexpr int kPitch = 272, kSlice = 32 * kPitch;
    const int r_lo = row & 31, wv = (row >> 5) & (NW - 1);
    uint8_t* stg = ostg + wv * kSlice;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x16& a = oacc[db];
        u32x2 w = {pack_bf16x2(a[4 * jj] * f, a[4 * jj + 1] * f),
                   pack_bf16x2(a[4 * jj + 2] * f, a[4 * jj + 3] * f)};
        *reinterpret_cast<u32x2*>(stg + r_lo * kPitch + (db * 32 + 8 * jj + 4 * g) * 2) = w;
      }
    if (g == 0 && lse != nullptr && row < Nq)
      lse[(int64_t)bh * Nq + row] =
          (m_run + log2f(lt) - (MODE == 2 ? 0.0f : kLog2PScale)) * kLn2;
    wave_lds_sync();
    debug_sync();
    // Store kk covers rows 4kk .. 4kk+3 of the wave; lane = 16 * (row % 4) + chunk.
    const int row0 = row - r_lo, sub = 2 * g + (r_lo >> 4), ch = r_lo & 15;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int r = 4 * kk + sub;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stg + r * kPitch + ch * 16);
      if (row0 + r < Nq)
        *reinterpret_cast<u32x4*>(o + q_base + (int64_t)(row0 + r) * D + ch * 8) = val;
    }
  } else if (row < Nq) {
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
      lse[(int64_t)bh * Nq + row] =
          (m_run + log2f(lt) - (MODE == 2 ? 0.0f : kLog2PScale)) * kLn2;
  }
}

template <int D, int NW, int MODE>
static int launch_fp8(const void* q8, const void* k8, const void* v8,
                      const float* descale, const void* q_e8, const void* k_e8,
                      const void* v_e8, void* o,
                      float* lse, int B, int H, int Nq, int Nkv, float scale,
                      hipStream_t stream) {
  using C = Fp8Cfg<D, NW>;
  const int n_qt = (Nq + C::kBM - 1) / C::kBM;
  const int64_t grid = (int64_t)n_qt * B * H;
  if (grid > 0x7FFFFFFF) return DTA_EUNSUPPORTED;
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, NW, MODE>), dim3((unsigned)grid),
                     dim3(C::kThreads), 0, stream,
                     static_cast<const uint8_t*>(q8), static_cast<const uint8_t*>(k8),
                     static_cast<const uint8_t*>(v8), descale,
                     static_cast<const uint8_t*>(q_e8), static_cast<const uint8_t*>(k_e8),
                     static_cast<const uint8_t*>(v_e8), static_cast<uint16_t*>(o), lse, Nq, Nkv,
                     scale, n_qt);
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
    return launch_fp8<128, 8, 0>(q8, k8, v8, descale, nullptr, nullptr, nullptr, o, lse, B, H,
                                 Nq, Nkv, scale, stream);
  return launch_fp8<64, 4, 0>(q8, k8, v8, descale, nullptr, nullptr, nullptr, o, lse, B, H, Nq,
                              Nkv, scale, stream);
}

extern "C" int attn_fwd_fp8_rows(const void* q8, const void* k8, const void* v8,
                                 const void* q_e8m0, const void* k_e8m0,
                                 const float* v_descale, void* o, float* lse, int B, int H,
                                 int Nq, int Nkv, int D, float scale, hipStream_t stream) {
  if (!q8 || !k8 || !v8 || !q_e8m0 || !k_e8m0 || !v_descale || !o) return DTA_EINVAL;
  if (B < 1 || H < 1 || Nq < 1 || Nkv < 1) return DTA_EINVAL;
  if (!(scale >= 0.f) || !__builtin_isfinite(scale)) return DTA_EINVAL;
  if (D != 64 && D != 128) return DTA_EUNSUPPORTED;
  auto al = [](const void* p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
  };
  if (!al(q8, 16) || !al(k8, 16) || !al(v8, 16) || !al(o, 16) || !al(v_descale, 4) ||
      (lse && !al(lse, 4)))
    return DTA_EALIGN;
  if (D == 128)
    return launch_fp8<128, 8, 1>(q8, k8, v8, v_descale, q_e8m0, k_e8m0, nullptr, o, lse, B, H,
                                 Nq, Nkv, scale, stream);
  return launch_fp8<64, 4, 1>(q8, k8, v8, v_descale, q_e8m0, k_e8m0, nullptr, o, lse, B, H, Nq,
                              Nkv, scale, stream);
}

extern "C" int attn_fwd_fp8_rows_v(const void* q8, const void* k8, const void* v8,
                                   const void* q_e8m0, const void* k_e8m0, const void* v_e8m0,
                                   void* o, float* lse, int B, int H, int Nq, int Nkv, int D,
                                   float scale, hipStream_t stream) {
  if (!q8 || !k8 || !v8 || !q_e8m0 || !k_e8m0 || !v_e8m0 || !o) return DTA_EINVAL;
  if (B < 1 || H < 1 || Nq < 1 || Nkv < 1) return DTA_EINVAL;
  if (!(scale >= 0.f) || !__builtin_isfinite(scale)) return DTA_EINVAL;
  if (D != 64 && D != 128) return DTA_EUNSUPPORTED;
  auto al = [](const void* p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
  };
  if (!al(q8, 16) || !al(k8, 16) || !al(v8, 16) || !al(o, 16) || (lse && !al(lse, 4)))
    return DTA_EALIGN;
  if (D == 128)
    return launch_fp8<128, 4, 2>(q8, k8, v8, nullptr, q_e8m0, k_e8m0, v_e8m0, o, lse, B, H, Nq,
                                 Nkv, scale, stream);
  return launch_fp8<64, 4, 2>(q8, k8, v8, nullptr, q_e8m0, k_e8m0, v_e8m0, o, lse, B, H, Nq,
                              Nkv, scale, stream);
}
