// attn_fwd: non-causal multi-head attention forward, bf16 in, bf16 O and
// float32 natural-log LSE out, for gfx950 (CDNA4).
//
// Operation: O_i = sum_j exp(s_ij) v_j / sum_j exp(s_ij), s_ij = scale q_i.k_j,
// LSE_i = ln sum_j exp(s_ij) -- the attention every SDPA backend computes
// (diffusers "Accelerate inference" guide, section "Scaled dot product
// attention"), evaluated by tiles with an online softmax, which rearranges
// the same sums exactly.
//
// Design (one workgroup = NW waves = NW*32 query rows of one (b, h)):
// * Scores are computed transposed, S^T = K . Q^T, on
//   v_mfma_f32_32x32x16_bf16: K rows come from LDS as the A operand and the
//   wave's 32 Q rows stay in registers as the B operand for the whole K/V
//   loop. In the 32x32 accumulator layout lane l then owns query l%32 and 16
//   of every 32 keys (rows 8*(r/4) + 4*(l/32) + r%4 of register r), so the row
//   max and row sum are in-lane work plus one v_permlane32_swap between the
//   two wave halves.
// * O is accumulated transposed too, O^T += V^T . P^T: the exponentiated
//   scores, rounded to bf16, are the B operand straight from the registers
//   that held S^T. The V^T operand is read from the row-major V tile with
//   ds_read_b64_tr_b16, whose 16-lane 4x4 transposes hand each lane 4 keys of
//   one head dimension; two such reads cover exactly the 8 keys the lane's P
//   operand holds, so no shuffle of P is needed.
// * K and V tiles (BN keys) are double-buffered in LDS with padded rows: a
//   16-byte pad puts the 16 K rows one 128-bit read quarter-wave touches in
//   distinct bank groups, a 64-byte pad does the same for the 4 rows x 64
//   bytes a half-wave of transposing V reads touches. Every operand address
//   is then a per-lane base plus an immediate. The next tile's global loads
//   are issued before the current tile's MFMAs and stored to the other buffer
//   after them: one barrier per tile.
// * For D = 128 a workgroup has 8 waves (256 query rows, one workgroup per CU
//   at two waves per SIMD): every K/V tile staged through registers and
//   written to LDS then feeds twice as many MFMAs as with 4 waves. LDS write
//   and global-load issue were the scarce resources at 4 waves (2 workgroups
//   per CU each staging its own copy of the tile); this is 12-17% faster.
// * Softmax runs in the log2 domain with c = scale*log2(e) folded into one FMA
//   per score before v_exp_f32. The running max used for the exponent is only
//   raised when some row's max grows by more than kTau (log2 units), so the
//   O accumulator is rescaled rarely; p stays below 2^kTau, and O and l share
//   the same reference max, so the result is exact.
// * Only the last, partial K/V tile masks keys; its rows past Nkv fail the
//   buffer range check, read as zero and get zero weight.
// * Workgroup ids are remapped so that the workgroups of one XCD walk
//   consecutive query tiles of the same head and share K/V through its L2.

#include <type_traits>

#include "common.h"

namespace dta {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D, int NW, int BN>
struct AttnCfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kBM = NW * 32;               // query rows per workgroup
  static constexpr int kCPR = D / 8;                // 16-byte chunks per row
  static constexpr int kRP = 16 / kCPR;             // rows per 256 bytes
  static constexpr int kKS = D + 8;                 // K row stride (elements)
  static constexpr int kVS = D + 32;                // V row stride (elements)
  static constexpr int kChunks = BN * kCPR;         // chunks per tile
  static constexpr int kCpt = kChunks / kThreads;   // chunks per thread
  static_assert(kChunks % kThreads == 0, "tile must split evenly");
  static_assert(BN % 32 == 0 && (D == 64 || D == 128), "tile shape");
};

constexpr float kTau = 8.0f;
// Fourth dword of a raw buffer resource (32-bit data format, no swizzle).
constexpr int kBufDword3 = 0x00020000;

__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ACCUM: instead of writing this K/V chunk's (O, LSE), merge it into the
// running (O, LSE) already in o / lse (one ring-attention step, fused).
template <int D, int NW, int BN, bool ACCUM>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int Nq, int Nkv, float c, int n_qt) {
  using C = AttnCfg<D, NW, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BN * C::kKS];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][BN * C::kVS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = blk / n_qt, qt = blk - bh * n_qt;
  const int64_t q_base = (int64_t)bh * Nq * D;
  const uint16_t* kh = k + (int64_t)bh * Nkv * D;
  const uint16_t* vh = v + (int64_t)bh * Nkv * D;
  const int row = qt * C::kBM + wave * 32 + l32;

  // Q^T operand: query `row`, dims ds*16 + 8g .. +7.
  bf16x8 qr[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds)
    qr[ds] = (row < Nq) ? *reinterpret_cast<const bf16x8*>(q + q_base + (int64_t)row * D +
                                                           ds * 16 + g * 8)
                        : bf16x8{};

  // Tile staging: chunk ci -> row ci / kCPR, logical chunk ci % kCPR; 16
  // consecutive threads cover 256 contiguous bytes of global memory. Loads go
  // through buffer resources whose base and byte range are the tile's: the
  // per-lane offsets stay constant, the address arithmetic is scalar, and rows
  // past Nkv fail the range check and read as zero.
  u32x4 kreg[C::kCpt], vreg[C::kCpt];
  const int st_r = tid / C::kCPR, st_c = tid % C::kCPR;   // row/chunk of it = 0
  constexpr int kRowsPerIt = C::kThreads / C::kCPR;
  auto load_tile = [&](int j) {
    const int64_t key0 = (int64_t)j * BN;
    const int bytes = (int)min<int64_t>((int64_t)(Nkv - key0) * D * 2, (int64_t)BN * D * 2);
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kh + key0 * D), 0, bytes, kBufDword3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vh + key0 * D), 0, bytes, kBufDword3);
#pragma unroll
    for (int it = 0; it < C::kCpt; ++it) {
      const int off = ((st_r + it * kRowsPerIt) * D + st_c * 8) * 2;
      kreg[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0);
      vreg[it] = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < C::kCpt; ++it) {
      const int r = st_r + it * kRowsPerIt;
      *reinterpret_cast<u32x4*>(&ks[buf][r * C::kKS + st_c * 8]) = kreg[it];
      *reinterpret_cast<u32x4*>(&vs[buf][r * C::kVS + st_c * 8]) = vreg[it];
    }
  };

  // Per-lane bases of the operand reads; everything else is an immediate.
  const int k_base = l32 * C::kKS + g * 8;
  const int v_base = (4 * g + ((lane & 15) >> 2)) * C::kVS +
                     16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int n_tiles = (Nkv + BN - 1) / BN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  // One K/V tile: MASK is set only for the last tile when Nkv % BN != 0.
  auto tile = [&](int j, auto buf_tag, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int buf = decltype(buf_tag)::value;
    const bool has_next = j + 1 < n_tiles;
    if (has_next) load_tile(j + 1);
    const uint16_t* kt = ks[buf];
    const uint16_t* vt = vs[buf];

    // S^T = K . Q^T, BN keys x 32 queries. The K fragments of step ds+1 are
    // read while the MFMAs of step ds run.
    f32x16 s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) s[kb] = f32x16{};
    bf16x8 kf[2][BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
      kf[0][kb] = *reinterpret_cast<const bf16x8*>(kt + k_base + kb * 32 * C::kKS);
    __builtin_amdgcn_sched_group_barrier(0x100, BN / 32, 0);
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      if (ds + 1 < D / 16) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
          kf[(ds + 1) & 1][kb] = *reinterpret_cast<const bf16x8*>(
              kt + k_base + kb * 32 * C::kKS + (ds + 1) * 16);
        __builtin_amdgcn_sched_group_barrier(0x100, BN / 32, 0);
      }
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds & 1][kb], qr[ds], s[kb], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, BN / 32, 0);
    }

    // Online softmax in the log2 domain.
    const int key_lim = Nkv - j * BN;
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3) >= key_lim) s[kb][r] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = xhalf_max(mx) * c;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kTau) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    float rs = 0.f;
    bf16x8 pb[BN / 32][2];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * t + i;
          p[i] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m_run));
          if constexpr (MASK) {
            if (kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3) >= key_lim) p[i] = 0.f;
          }
          rs += p[i];
        }
        pb[kb][t] = bf16x8{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                           (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
        // Keep the row sum next to the exponentials: the float32 p values
        // then die here instead of living across the P.V MFMAs.
        asm volatile("" : "+v"(rs));
      }
    l_run += rs;

    // O^T += V^T . P^T, 16 keys per MFMA; V^T via transposing LDS reads.
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          s16x4 part[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int off = v_base + (kb * 32 + 16 * t + 8 * h) * C::kVS + db * 32;
            part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + off));
          }
          const s16x4 lo = part[0], hi = part[1];
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3],
                                                                   hi[0], hi[1], hi[2], hi[3]});
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][t], oacc[db], 0, 0, 0);
        }

    debug_sync();
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  const int n_full = (Nkv % BN == 0) ? n_tiles : n_tiles - 1;
  int j = 0;
  for (; j + 1 < n_full; j += 2) {
    tile(j, B0{}, std::false_type{});
    tile(j + 1, B1{}, std::false_type{});
  }
  if (j < n_full) tile(j++, B0{}, std::false_type{});
  if (j < n_tiles) {
    if (j & 1)
      tile(j, B1{}, std::true_type{});
    else
      tile(j, B0{}, std::true_type{});
  }

  // Epilogue: lane owns query `row` and dims db*32 + 8*(r/4) + 4g + r%4.
  const float lt = xhalf_sum(l_run);
  const int64_t li = (int64_t)bh * Nq + row;
  if constexpr (D == 128 && NW == 8) {
    debug_sync();
    // O goes through LDS so that the global loads and stores of O are whole
    // 256-byte rows (16 lanes per row) instead of 16 bytes of each of 32
    // rows per instruction. The last tile's barrier has retired every K/V
    // read; each wave uses its own slice of the K/V buffers (32 rows at a
    // 272-byte pitch, conflict-free 8-byte accesses) and touches no other
    // slice, so no further barrier is needed. Every lane takes part: the rows
    // a lane loads and stores are not its own. The indices derive from `row`
    // and `g` alone, which keeps the loop's register allocation as without
    // this epilogue.
    constexpr int kPitch = 272, kSlice = 32 * kPitch;
    static_assert(sizeof(ks) >= 4 * kSlice && sizeof(vs) >= 4 * kSlice, "O staging");
    const int r_lo = row & 31, wv = (row >> 5) & 7;
    uint8_t* stg = wv < 4 ? reinterpret_cast<uint8_t*>(&ks[0][0]) + wv * kSlice
                          : reinterpret_cast<uint8_t*>(&vs[0][0]) + (wv - 4) * kSlice;
    // Coalesced access kk covers rows 4kk .. 4kk+3 of the wave; lane =
    // 16 * (row % 4) + 16-byte chunk.
    const int row0 = row - r_lo, sub = 2 * g + (r_lo >> 4), ch = r_lo & 15;
    if constexpr (!ACCUM) {
      const float inv = 1.0f / lt;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x16& a = oacc[db];
          u32x2 w = {pack_bf16x2(a[4 * jj] * inv, a[4 * jj + 1] * inv),
                     pack_bf16x2(a[4 * jj + 2] * inv, a[4 * jj + 3] * inv)};
          *reinterpret_cast<u32x2*>(stg + r_lo * kPitch + (db * 32 + 8 * jj + 4 * g) * 2) = w;
        }
      if (g == 0 && lse != nullptr && row < Nq) lse[li] = (m_run + log2f(lt)) * kLn2;
    } else {
      // The running O rows into the slice, then the two-part merge below in
      // place there (rows past Nq hold zeros and are never stored).
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int r = 4 * kk + sub;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (row0 + r < Nq)
          val = *reinterpret_cast<const u32x4*>(o + q_base + (int64_t)(row0 + r) * D + ch * 8);
        *reinterpret_cast<u32x4*>(stg + r * kPitch + ch * 16) = val;
      }
      wave_lds_sync();
      debug_sync();
      // Two-part log-sum-exp merge in the log2 domain, as below.
      const float lc = m_run + log2f(lt);
      const float lr = row < Nq ? lse[li] * kLog2e : -INFINITY;
      const float mm = fmaxf(lc, lr);
      const float wr = __builtin_amdgcn_exp2f(lr - mm);
      const float wc = __builtin_amdgcn_exp2f(lc - mm);
      const float den = wr + wc;
      const float ar = wr / den;
      const float ac = wc / (den * lt);
      const bool use_r = wr > 0.f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          uint8_t* cell = stg + r_lo * kPitch + (db * 32 + 8 * jj + 4 * g) * 2;
          const u32x2 prev = *reinterpret_cast<const u32x2*>(cell);
          const f32x16& a = oacc[db];
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t wv2 = prev[e >> 1];
            const float orv = bf16_bits_to_f32((e & 1) ? (wv2 >> 16) : (wv2 & 0xFFFF));
            x[e] = a[4 * jj + e] * ac + (use_r ? orv * ar : 0.f);
          }
          *reinterpret_cast<u32x2*>(cell) =
              u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        }
      if (g == 0 && row < Nq) lse[li] = (mm + log2f(den)) * kLn2;
    }
    wave_lds_sync();
    debug_sync();
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int r = 4 * kk + sub;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stg + r * kPitch + ch * 16);
      if (row0 + r < Nq)
        *reinterpret_cast<u32x4*>(o + q_base + (int64_t)(row0 + r) * D + ch * 8) = val;
    }
    return;
  }
  if (row >= Nq) return;
  uint16_t* orow = o + q_base + (int64_t)row * D;
  if constexpr (!ACCUM) {
    const float inv = 1.0f / lt;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x16& a = oacc[db];
        u32x2 w = {pack_bf16x2(a[4 * jj] * inv, a[4 * jj + 1] * inv),
                   pack_bf16x2(a[4 * jj + 2] * inv, a[4 * jj + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * jj + 4 * g) = w;
      }
    if (g == 0 && lse != nullptr) lse[li] = (m_run + log2f(lt)) * kLn2;
  } else {
    // Two-part log-sum-exp merge in the log2 domain: the running part (O_r,
    // L_r) from memory and this chunk's (acc / lt, m_run + log2 lt). A running
    // L_r of -inf means "nothing seen yet": weight 0, and O_r is not used.
    const float lc = m_run + log2f(lt);
    const float lr = lse[li] * kLog2e;
    const float mm = fmaxf(lc, lr);
    const float wr = __builtin_amdgcn_exp2f(lr - mm);
    const float wc = __builtin_amdgcn_exp2f(lc - mm);
    const float den = wr + wc;
    const float ar = wr / den;
    const float ac = wc / (den * lt);
    const bool use_r = wr > 0.f;
    u32x2 prev[D / 32][4];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        prev[db][jj] = *reinterpret_cast<const u32x2*>(orow + db * 32 + 8 * jj + 4 * g);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x16& a = oacc[db];
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wv = prev[db][jj][e >> 1];
          const float orv = bf16_bits_to_f32((e & 1) ? (wv >> 16) : (wv & 0xFFFF));
          x[e] = a[4 * jj + e] * ac + (use_r ? orv * ar : 0.f);
        }
        const u32x2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * jj + 4 * g) = w;
      }
    if (g == 0) lse[li] = (mm + log2f(den)) * kLn2;
  }
}

template <int D, int NW, int BN, bool ACCUM>
static int launch_attn_fwd(const void* q, const void* k, const void* v,
                           void* o, float* lse, int B, int H, int Nq, int Nkv,
                           float scale, hipStream_t stream) {
  using C = AttnCfg<D, NW, BN>;
  const int n_qt = (Nq + C::kBM - 1) / C::kBM;
  const int64_t grid = (int64_t)n_qt * B * H;
  if (grid > 0x7FFFFFFF) return DTA_EUNSUPPORTED;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW, BN, ACCUM>), dim3((unsigned)grid),
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

// Argument checks shared by attn_fwd and attn_fwd_accum.
static int check_attn_args(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, int B, int H, int Nq, int Nkv, int D,
                           float scale) {
  if (!q || !k || !v || !o) return DTA_EINVAL;
  if (B < 1 || H < 1 || Nq < 1 || Nkv < 1) return DTA_EINVAL;
  if (!(scale >= 0.f) || !__builtin_isfinite(scale)) return DTA_EINVAL;
  if (D != 64 && D != 128) return DTA_EUNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return DTA_EALIGN;
  return DTA_OK;
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o,
                        float* lse, int B, int H, int Nq, int Nkv, int D,
                        float scale, hipStream_t stream) {
  const int st = check_attn_args(q, k, v, o, lse, B, H, Nq, Nkv, D, scale);
  if (st != DTA_OK) return st;
  if (D == 128)
    return launch_attn_fwd<128, 8, 64, false>(q, k, v, o, lse, B, H, Nq, Nkv, scale, stream);
  return launch_attn_fwd<64, 4, 64, false>(q, k, v, o, lse, B, H, Nq, Nkv, scale, stream);
}

extern "C" int attn_fwd_accum(const void* q, const void* k, const void* v, void* o,
                              float* lse, int B, int H, int Nq, int Nkv, int D,
                              float scale, hipStream_t stream) {
  if (!lse) return DTA_EINVAL;
  const int st = check_attn_args(q, k, v, o, lse, B, H, Nq, Nkv, D, scale);
  if (st != DTA_OK) return st;
  if (D == 128)
    return launch_attn_fwd<128, 8, 64, true>(q, k, v, o, lse, B, H, Nq, Nkv, scale, stream);
  return launch_attn_fwd<64, 4, 64, true>(q, k, v, o, lse, B, H, Nq, Nkv, scale, stream);
}
