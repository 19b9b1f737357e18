/*
 * dta.h -- C ABI of libdta.so, the MI355X (gfx950) diffusion-transformer
 * attention core.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is DEVICE memory owned by the caller. The library
 *   never allocates, frees or synchronises; each call only enqueues kernels on
 *   `stream` (0 = the null stream) and returns. Errors raised by the kernels
 *   themselves surface at the caller's next synchronisation, as usual in HIP.
 * - Layouts are dense row-major with 64-bit element offsets:
 *   Q [B,H,Nq,D], K and V [B,H,Nkv,D], O [B,H,Nq,D], LSE [B,H,Nq].
 * - Arguments are validated before any HIP call; a bad argument returns a
 *   negative dta_status and enqueues nothing. Only DTA_ELAUNCH can follow a
 *   HIP call. No function throws across the ABI.
 * - bf16 means IEEE-style bfloat16 (1-8-7) stored as uint16; fp8 means OCP
 *   E4M3FN bytes (bias 7, no infinities, max finite 448).
 * - Two calls that share one workspace `ws` must not run concurrently (on
 *   two streams); calls on one stream are ordered and may share it. A
 *   workspace is dta_ws_bytes() bytes of device memory, zero-filled once
 *   before its first use; every call leaves it fit for the next one.
 */
#ifndef DTA_H_
#define DTA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DTA_OK = 0,
  DTA_EINVAL = -1,        /* null pointer, non-positive size, bad scale      */
  DTA_EUNSUPPORTED = -2,  /* a head dimension other than 64 or 128           */
  DTA_EALIGN = -3,        /* a pointer not aligned as documented             */
  DTA_ELAUNCH = -4        /* the HIP runtime refused the kernel launch       */
} dta_status;

/*
 * attn_fwd -- non-causal multi-head scaled-dot-product attention, bf16 in,
 * bf16 O and float32 natural-log LSE out.
 *
 * Defines (diffusers "Accelerate inference" guide, section "Scaled dot
 * product attention"; no mask, no dropout, as the "Context parallelism"
 * guide, section "Ring Anything Attention", requires):
 *     s_ij = scale * q_i . k_j
 *     O_i  = sum_j exp(s_ij) v_j / sum_j exp(s_ij)      (rounded to bf16)
 *     LSE_i = ln sum_j exp(s_ij)                          (float32)
 * Called on one contiguous K/V chunk it produces that chunk's partial
 * (O, LSE), the local work of one ring-attention step (same guide, section
 * "Ring Attention"); attn_merge then combines the partials.
 *
 * q        bf16 [B,H,Nq,D], 16-byte aligned
 * k, v     bf16 [B,H,Nkv,D], 16-byte aligned
 * o        bf16 [B,H,Nq,D], 16-byte aligned, written
 * lse      float [B,H,Nq], 4-byte aligned, written (may be NULL: not written)
 * B,H,Nq,Nkv >= 1; D in {64, 128}; scale finite and >= 0 (1/sqrt(D) is usual)
 * Returns DTA_OK, DTA_EINVAL, DTA_EUNSUPPORTED, DTA_EALIGN or DTA_ELAUNCH.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Nq, int Nkv, int D, float scale,
             hipStream_t stream);

/*
 * attn_merge -- combine partial (O_p, LSE_p), p = 0..n_parts-1, computed by
 * attn_fwd over disjoint K/V chunks, into attention over their union:
 *     M = max_p LSE_p;  w_p = exp(LSE_p - M);  W = sum_p w_p
 *     O = sum_p w_p O_p / W  (bf16);  LSE = M + ln W  (float32)
 * This is the exact log-sum-exp identity behind ring attention, where every
 * rank has seen all tokens' K/V after a full turn (diffusers "Context
 * parallelism" guide, sections "Ring Attention" and "Ring Anything
 * Attention"). A partial with LSE = -inf gets zero weight; a row whose
 * partials are all -inf gets O = 0 and LSE = -inf. Arithmetic is float32.
 *
 * o_parts   bf16 [n_parts,B,H,Nq,D] packed, 16-byte aligned
 * lse_parts float [n_parts,B,H,Nq] packed, 4-byte aligned
 * o         bf16 [B,H,Nq,D], 16-byte aligned, written (must not alias inputs)
 * lse       float [B,H,Nq], written (may be NULL)
 * n_parts >= 1; B,H,Nq >= 1; D in {64, 128}.
 */
int attn_merge(const void* o_parts, const float* lse_parts, int n_parts,
               void* o, float* lse, int B, int H, int Nq, int D,
               hipStream_t stream);

/*
 * attn_fwd_accum -- one ring-attention step with the merge fused into the
 * attention epilogue (diffusers "Context parallelism" guide, section "Ring
 * Attention": each rank folds every K/V block it receives into its running
 * output). With (O_r, L_r) the running state held in o / lse and (O_c, L_c)
 * what attn_fwd would return for this K/V chunk, o / lse are overwritten in
 * place with the two-part attn_merge of the pair:
 *     M = max(L_r, L_c);  w_r = exp(L_r - M), w_c = exp(L_c - M)
 *     O = (w_r O_r + w_c O_c) / (w_r + w_c);  LSE = M + ln(w_r + w_c)
 * O_c is never rounded: the merge takes the float32 accumulator; only the
 * merged O is rounded to bf16, once per call (so a ring of n steps rounds the
 * running O n times, where attn_fwd + attn_merge round each partial once and
 * the merged O once). A row with L_r = -inf is "nothing seen yet": its O_r is
 * ignored (it may hold anything, NaN included) and the row receives the
 * chunk's result. Typical use: the first step calls attn_fwd (or starts from
 * lse filled with -inf), later steps call attn_fwd_accum on the same o / lse.
 * Steps on one (o, lse) must be ordered (one stream).
 *
 * q, k, v, B, H, Nq, Nkv, D, scale   as attn_fwd
 * o     bf16 [B,H,Nq,D], 16-byte aligned, read and written
 * lse   float [B,H,Nq], 4-byte aligned, read and written; must not be NULL;
 *       entries finite or -inf
 * Returns DTA_OK, DTA_EINVAL, DTA_EUNSUPPORTED, DTA_EALIGN or DTA_ELAUNCH.
 */
int attn_fwd_accum(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int H, int Nq, int Nkv, int D,
                   float scale, hipStream_t stream);

/*
 * attn_merge_into -- the pairwise, in-place form of attn_merge, for a
 * partial that arrives already computed (same guide and section):
 *     (o, lse) <- attn_merge of {(o, lse), (o_part, lse_part)}
 * A part with LSE = -inf gets zero weight and its O is ignored; a row whose
 * two LSEs are both -inf gets O = 0 and LSE = -inf. Arithmetic is float32,
 * the result is rounded to bf16 once.
 *
 * o         bf16 [B,H,Nq,D], 16-byte aligned, read and written
 * lse       float [B,H,Nq], 4-byte aligned, read and written (not NULL)
 * o_part    bf16 [B,H,Nq,D], 16-byte aligned (must not alias o)
 * lse_part  float [B,H,Nq], 4-byte aligned (not NULL)
 * B,H,Nq >= 1; D in {64, 128}.
 */
int attn_merge_into(void* o, float* lse, const void* o_part,
                    const float* lse_part, int B, int H, int Nq, int D,
                    hipStream_t stream);

/*
 * residual_diff -- First Block Cache's relative residual difference
 * (ParaAttention guide, section "First Block Cache"):
 *     out = sum_k |a_k - b_k| / sum_k |b_k|  ( = mean|a-b| / mean|b| )
 * over all n elements; a is the current step's first-block residual, b the
 * previous step's. Per-thread float32 partial sums, a fixed-order float64
 * finish, so the result is bitwise reproducible. sum|b| = 0 gives the IEEE
 * quotient (+inf or NaN). The threshold compare is the caller's, or
 * fbcache_step's, which fuses it with the cached-residual apply.
 * Enqueues one kernel: every workgroup writes its partial sums to ws, and
 * the last workgroup to finish adds them up and writes out.
 *
 * a, b  bf16 [n], 16-byte aligned; n >= 1
 * out   float, one device scalar, written
 * ws    device workspace of at least dta_ws_bytes() bytes, 16-byte aligned,
 *       zero-filled once before its first use (it holds the per-workgroup
 *       partials and an arrival counter that each call returns to zero).
 */
int residual_diff(const void* a, const void* b, int64_t n, float* out,
                  void* ws, hipStream_t stream);

/*
 * residual_diff_noalloc -- residual_diff for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernel and the same result, bit for bit, with the
 * workspace replaced by a scratch array inside the library. The call
 * allocates nothing and frees nothing.
 *
 * The scratch is a fixed 20 736-byte device array per GPU, held until the
 * process ends; it holds the fixed grid's 512 partial pairs and the arrival
 * counters, so its size does not depend on n. Every call on one GPU shares
 * it: calls that overlap on one GPU (two streams, or two host threads) race
 * and must not be issued. Each call returns the counters to zero.
 * a, b  bf16 [n], 16-byte aligned; 1 <= n < 2^62 (beyond that DTA_EINVAL)
 * out   float, one device scalar, written
 * stream  a stream of the current device (or 0); another device's stream
 *         gives DTA_EINVAL. The first call on a device looks up the
 *         scratch's address there (a failure gives DTA_ELAUNCH).
 */
int residual_diff_noalloc(const void* a, const void* b, int64_t n, float* out,
                          hipStream_t stream);

/*
 * fbcache_step -- First Block Cache's decision and cached-residual apply on
 * the device, with no host round trip (ParaAttention guide, section "First
 * Block Cache": when the first block's relative residual difference is small
 * enough the step skips the remaining blocks and reuses their cached
 * residual; 0.08 is FLUX's default threshold):
 *     diff = sum|r - r_prev| / sum|r_prev|           (exactly residual_diff)
 *     use  = diff < threshold                          (float32 compare; a NaN
 *                                                      diff never reuses)
 *     if use:  hidden[i] = bf16(hidden[i] + cached[i])  (float32 sum, rounded
 *                                                      once, to nearest even)
 * `use` is written to *use_cache (0 or 1) for later device-side work; hidden
 * is untouched when it is 0. Enqueues two kernels: residual_diff's (whose
 * last workgroup also takes the decision) and the apply (whose workgroups
 * leave at once when use = 0).
 *
 * r, r_prev   bf16 [n], 16-byte aligned; n >= 1 (this and the previous
 *             step's first-block residual)
 * hidden      bf16 [n_hidden], 16-byte aligned, read and written
 * cached      bf16 [n_hidden], 16-byte aligned (must not alias hidden)
 * diff        float, device scalar, written;  use_cache  int, device, written
 * ws          as for residual_diff (not concurrently with another user)
 */
int fbcache_step(const void* r, const void* r_prev, int64_t n, float threshold,
                 void* hidden, const void* cached, int64_t n_hidden,
                 float* diff, int* use_cache, void* ws, hipStream_t stream);

/*
 * fp8_quant_per_tensor -- per-tensor dynamic quantisation to E4M3FN
 * (ParaAttention guide, section "fp8 quantization": one scale per tensor is
 * the default granularity):
 *     s = amax|x| / 448 in float32 (s = 1 if amax = 0)
 *     x8 = e4m3_rne(float32(x) / s)   (correctly rounded float32 division,
 *                                      round-to-nearest-even, saturating)
 * x        bf16 [n], 16-byte aligned; n >= 1
 * x8       uint8 [n], 16-byte aligned, written
 * descale  float, one device scalar, written with s
 * ws       as for residual_diff (may be the same buffer, not concurrently;
 *          the quantisers leave residual_diff's counter untouched)
 * Enqueues two kernels: partial maxima into ws, and the cast, every
 * workgroup of which reduces the partials itself; workgroup 0 writes
 * descale.
 */
int fp8_quant_per_tensor(const void* x, int64_t n, void* x8, float* descale,
                         void* ws, hipStream_t stream);

/*
 * fp8_quant_per_tensor_multi -- fp8_quant_per_tensor of up to four tensors
 * (typically Q, K and V of one attention call) in the same two launches:
 * one kernel writes every tensor's partial maxima, one casts every tensor.
 * Tensor t gets exactly the codes and scale fp8_quant_per_tensor gives it.
 * count    1..4
 * x, n, x8 HOST arrays of count entries: device pointers to bf16 [n[t]]
 *          (16-byte aligned), element counts n[t] >= 1, and device pointers
 *          to uint8 [n[t]] (16-byte aligned, written)
 * descale  device float[count], 4-byte aligned, written with the scales
 * ws       as for residual_diff (dta_ws_bytes() covers four tensors)
 * Returns DTA_OK, DTA_EINVAL (count out of range, a null pointer, a size
 * < 1), DTA_EALIGN or DTA_ELAUNCH.
 */
int fp8_quant_per_tensor_multi(int count, const void* const* x, const int64_t* n,
                               void* const* x8, float* descale, void* ws,
                               hipStream_t stream);

/*
 * attn_fwd_fp8 -- the fp8 dynamic-quantisation variant of attn_fwd: Q, K, V
 * are E4M3FN with per-tensor scales (as fp8_quant_per_tensor writes them);
 * S = scale * s_q s_k (Q8 . K8^T) on fp8 MFMA with float32 accumulation;
 * p = exp(s - m) is quantised to E4M3FN at x108 before the P.V product,
 * where m is the online softmax's reference max, kept within a factor 4 of
 * the running row max so that 108 p <= 432 (E4M3's largest value is 448);
 * O = (P8 . V8) s_v / (108 l) with l the float32 sum of the unquantised p;
 * LSE = m + ln l.
 *
 * q8, k8, v8  E4M3FN bytes, layouts as attn_fwd, 16-byte aligned
 * descale     device float[3] = {s_q, s_k, s_v}
 * o, lse      as attn_fwd. D in {64, 128}.
 */
int attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                 const float* descale, void* o, float* lse, int B, int H,
                 int Nq, int Nkv, int D, float scale, hipStream_t stream);

/*
 * Layout kernels of context parallelism (diffusers "Context parallelism"
 * guide): the local permutations on either side of the exchanges.
 * - Ulysses Attention: an all-to-all turns [B,H,n_rank,D] (all heads, this
 *   rank's tokens) into [B,H_rank,N,D] (this rank's heads, all tokens) and
 *   back. The sender splits along one axis into per-destination parts, the
 *   receiver concatenates the received parts along the other. Ulysses
 *   Anything Attention allows uneven parts on both axes.
 * - Ring Anything Attention: ranks hold uneven token counts; each part is
 *   padded to the longest for the all-gather and the padding is dropped when
 *   the gathered parts are concatenated.
 * Parts are stored back to back in one buffer, part p first. Sizes are HOST
 * arrays of P ints (1 <= P <= 64). Any D that is a multiple of 8 works
 * (rows move as 16-byte chunks); every element is bf16 / 2 bytes, so the
 * kernels copy any 16-bit payload exactly. Buffers must not overlap.
 *
 * seq_concat  parts: part p = [B,H,padded[p],D] whose first lens[p] tokens
 *             are valid; out = [B,H,sum lens,D], part p's tokens at offset
 *             lens[0]+...+lens[p-1]. padded NULL means padded = lens.
 *             lens[p] >= 0, padded[p] >= max(lens[p], 1), sum lens >= 1.
 * seq_split   the inverse: x = [B,H,sum lens,D] -> parts; tokens lens[p] ..
 *             padded[p]-1 of each part are written as zeros.
 * head_concat parts: part p = [B,heads[p],N,D]; out = [B,sum heads,N,D].
 * head_split  the inverse. heads[p] >= 1 for every part: a part with no
 *             heads is rejected (DTA_EINVAL), as is lens[p] = 0 with padded
 *             NULL (a part must occupy at least one row).
 * All are 16-byte aligned device buffers. Return DTA_OK, DTA_EINVAL (bad
 * sizes, P out of range, D not a multiple of 8), DTA_EALIGN or DTA_ELAUNCH.
 */
int seq_concat(const void* parts, void* out, int P, const int* lens,
               const int* padded, int B, int H, int D, hipStream_t stream);
int seq_split(const void* x, void* parts, int P, const int* lens,
              const int* padded, int B, int H, int D, hipStream_t stream);
int head_concat(const void* parts, void* out, int P, const int* heads, int B,
                int N, int D, hipStream_t stream);
int head_split(const void* x, void* parts, int P, const int* heads, int B,
               int N, int D, hipStream_t stream);

/*
 * fp8_quant_rows_pow2 -- row-wise dynamic quantisation to E4M3FN with one
 * power-of-two scale per row (ParaAttention guide, section "fp8
 * quantization": row-wise scaling as the more accurate alternative to the
 * per-tensor default). For Q and K a row is one token of one head (row_len
 * = D):
 *     e = the smallest integer with amax|row| <= 448 * 2^e, clamped to
 *         [-127, 127]; e = 0 for an all-zero row
 *     x8 = e4m3_rne(x * 2^-e)     (the scaling is exact)
 *     e8m0[row] = e + 127          (OCP E8M0 byte: the scale is 2^(byte-127))
 * E4M3 keeps 3 mantissa bits in every binade, so a power-of-two scale loses
 * nothing against amax/448; it only sets the saturation and underflow limits.
 * x finite bf16 [rows * row_len], 16-byte aligned; x8 uint8 same count,
 * 8-byte aligned; e8m0 uint8 [rows]. row_len a multiple of 8, rows >= 1.
 */
int fp8_quant_rows_pow2(const void* x, int64_t rows, int row_len, void* x8,
                        void* e8m0, hipStream_t stream);

/*
 * attn_fwd_fp8_rows -- attn_fwd_fp8 with row-wise power-of-two scales for Q
 * and K (as fp8_quant_rows_pow2 writes them, one E8M0 byte per token of each
 * head: q_e8m0 [B,H,Nq], k_e8m0 [B,H,Nkv]) and V per tensor (v_descale,
 * one device float, as fp8_quant_per_tensor writes it):
 *     s_ij = scale * 2^(eq_i + ek_j) (Q8_i . K8_j)
 * The exponents are applied by the fp8 MFMA's operand scales (a per-lane
 * scale for each key row of K and each query column of Q^T), so they cost
 * no VALU work. P, O and LSE are as in attn_fwd_fp8.
 */
int attn_fwd_fp8_rows(const void* q8, const void* k8, const void* v8,
                      const void* q_e8m0, const void* k_e8m0,
                      const float* v_descale, void* o, float* lse, int B, int H,
                      int Nq, int Nkv, int D, float scale, hipStream_t stream);

/*
 * attn_fwd_fp8_rows_v -- the row-wise variant with per-token power-of-two
 * scales for V as well, and per-block power-of-two scales for P
 * (ParaAttention guide, section "fp8 quantization": row-wise scaling as the
 * more accurate option).
 *   q8, k8, v8: E4M3 codes [B,H,Nq|Nkv,D], e.g. fp8_quant_rows_pow2 with
 *               row_len = D (device, 16-byte aligned);
 *   q_e8m0, k_e8m0, v_e8m0: one E8M0 byte per token, [B,H,Nq] / [B,H,Nkv]
 *               (device); the scale of a token is 2^(byte - 127);
 *   o: bf16 [B,H,Nq,D] (16-byte aligned); lse: float32 [B,H,Nq], or NULL.
 * Q and K scales act as in attn_fwd_fp8_rows. V's scale is folded into the
 * probabilities, pv_j = p_j 2^(ev_j - 127), with p_j = exp(s_j - m) against
 * the running row maximum; pv is quantised to E4M3 with one power-of-two scale
 * 2^e per (query, block of 32 consecutive keys), e the smallest integer with
 * max pv <= 448 * 2^e (clamped to [-126, 127]). That scale is the P.V MFMA's
 * operand scale, which the fp8 MFMA applies per 32 consecutive k.
 *     O_i = sum_j P^_ij V8_j / sum_j p_ij,  LSE_i = m_i + ln sum_j p_ij
 * with P^ the dequantised pv and V8 V's E4M3 values. Inside one block, pv
 * values more than E4M3's span (about 2^17) below the block's largest round
 * to zero. V exponent bytes must be <= 252 (p reaches 2^2 against the
 * running maximum, and pv must stay a finite float32); the exponents of any
 * bf16 or float32 tensor are (<= 247). Errors: DTA_EINVAL (a null pointer, a
 * size < 1, a negative or non-finite scale), DTA_EUNSUPPORTED (D other than
 * 64 or 128), DTA_EALIGN.
 */
int attn_fwd_fp8_rows_v(const void* q8, const void* k8, const void* v8,
                        const void* q_e8m0, const void* k_e8m0, const void* v_e8m0,
                        void* o, float* lse, int B, int H, int Nq, int Nkv, int D,
                        float scale, hipStream_t stream);

/* Bytes of the workspace residual_diff, fbcache_step and the per-tensor
 * quantisers need (zero-filled once before first use). */
size_t dta_ws_bytes(void);

/* A static, human-readable name of a dta_status value. */
const char* dta_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* DTA_H_ */
