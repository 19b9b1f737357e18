"""Oracle: per-tensor dynamic fp8 (OCP E4M3FN) quantisation and fp8 attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); never on the product
path.

ParaAttention guide, section "fp8 quantization": dynamic quantisation to fp8
lets 8-bit matrix units run; the default granularity is one scale per tensor
(per-row scales are the more accurate option where supported). The pages fix
neither the fp8 encoding nor the P handling, so these readings are taken:

* Format: OCP E4M3FN -- 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
  bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no
  infinity; the largest finite magnitude is 448.
* Per-tensor scale: s = amax|x| / 448 computed in float32 (s = 1 when
  amax = 0); code = e4m3(x / s) with the division in float32 and the
  rounding to E4M3 round-to-nearest-even, saturating at +-448.
* Attention on the dequantised values x^ = e4m3_value(code) * s, with the
  probabilities quantised before the P.V product: p = exp(s_ij - m_i) lies in
  (0, 1]; P8 = e4m3(448 p) uses the full E4M3 range; O = (P8 . V^) / (448 l)
  with l = sum_j p_ij taken from the unquantised p; LSE = m + ln l.
"""

import numpy as np

E4M3_MAX = 448.0
_E4M3_NAN = 0x7F


def e4m3_decode(codes):
    """Value of each E4M3FN byte as float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, subnormal, normal)
    val = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)
    return sign * val


# The 127 finite non-negative magnitudes, in code order 0x00 .. 0x7E. Codes
# are monotone in magnitude, so "nearest, ties to even mantissa" is "nearest,
# ties to the even code" along this table.
_MAGS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x):
    """Round each value to the nearest E4M3FN code (ties to even), saturating.

    Magnitudes at or above 448 map to +-448; NaN maps to 0x7F; the sign bit
    is kept for values that round to zero (-0.0 -> 0x80).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    hi = np.searchsorted(_MAGS, a, side="left")          # first mag >= a
    hi_c = np.minimum(hi, 0x7E)
    lo_c = np.maximum(hi_c - 1, 0)
    d_hi = _MAGS[hi_c] - a
    d_lo = a - _MAGS[lo_c]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))
    code = np.where(pick_hi, hi_c, lo_c)
    code = np.where(a == _MAGS[hi_c], hi_c, code)        # exact hit
    code = np.where(a >= E4M3_MAX, 0x7E, code)           # saturate
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(np.isnan(x), _E4M3_NAN, code)
    return code.astype(np.uint8)


def e4m3_round(x):
    """The float64 value of the E4M3FN number nearest to each x (ties to the
    even mantissa), saturating at +-448; NaN stays NaN. Equal to
    ``e4m3_decode(e4m3_encode(x))``, computed from the format's spacing
    instead of a table search: a binade [2^(e-1), 2^e) at or above 2^-6
    holds 8 values 2^(e-4) apart (3 mantissa bits), and below 2^-6 the
    subnormals are 2^-9 apart, so the nearest value is an integer multiple
    of that spacing (numpy's round is half-to-even, and an even multiple is
    an even mantissa, also where a tie rounds up into the next binade).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                       # a in [2^(e-1), 2^e)
    spacing = np.ldexp(1.0, np.maximum(e - 4, -9))
    with np.errstate(invalid="ignore"):
        r = np.minimum(np.round(a / spacing) * spacing, E4M3_MAX)
    return np.where(np.isnan(x), np.nan, np.copysign(r, x))


def quant_per_tensor(x):
    """Per-tensor dynamic quantisation of ``x`` to E4M3FN.

    Returns (codes: uint8 array of x's shape, s: the float32 scale as a Python
    float) with s = amax|x|/448 in float32 (1 if amax = 0) and
    codes = e4m3(float32(x) / s), the division correctly rounded in float32.
    """
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float32).numpy()
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.abs(x32).max()) if x32.size else np.float32(0)
    if amax == 0:
        s = np.float32(1.0)
    else:
        s = np.float32(amax / np.float32(E4M3_MAX))
    y = (x32 / s).astype(np.float32)
    return e4m3_encode(y.astype(np.float64)), float(s)


def attention_fp8(q8, k8, v8, descale, scale, rows=None):
    """Attention on per-tensor E4M3 inputs with P quantised to E4M3 at x448.

    q8: [B,H,Nq,D] uint8 codes, k8/v8: [B,H,Nkv,D] uint8 codes,
    descale: (s_q, s_k, s_v), scale: logit multiplier, rows: optional query
    rows. Returns (O, LSE) in float64, shapes as ``oracle.attention``.
    """
    q = e4m3_decode(np.asarray(q8)) * float(descale[0])
    k = e4m3_decode(np.asarray(k8)) * float(descale[1])
    v = e4m3_decode(np.asarray(v8)) * float(descale[2])
    return _attention_p8(q, k, v, scale, rows)


def pow2_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127];
    0 where amax == 0. Exact: amax = m * 2^k with 0.5 <= m < 1 (frexp) and
    448 = 0.875 * 2^9, so amax <= 448 * 2^e iff e >= k - 9 when m <= 0.875,
    else e >= k - 8."""
    amax = np.asarray(amax, dtype=np.float64)
    m, k = np.frexp(amax)
    e = np.where(m <= 0.875, k - 9, k - 8)
    return np.where(amax == 0, 0, np.clip(e, -127, 127)).astype(np.int64)


def quant_rows_pow2(x, row_len):
    """Row-wise dynamic quantisation to E4M3FN with power-of-two scales.

    ParaAttention guide, section "fp8 quantization": per-tensor scaling is
    the default and row-wise scaling the more accurate option. Each row of
    ``row_len`` consecutive elements (one token of one head for Q and K) gets
    its own scale 2^e with e the smallest integer such that amax_row <=
    448 * 2^e, clamped to [-127, 127] (e = 0 for an all-zero row); codes are
    e4m3(x * 2^-e), the scaling exact. A power of two loses nothing against
    amax/448: E4M3 keeps 3 mantissa bits in every binade, so only the
    saturation and underflow limits depend on the scale, and these are set
    the same way. Returns (codes uint8 of x's shape, exponents as E8M0 bytes
    e + 127, one per row).
    """
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float32).numpy()
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    if row_len < 1 or x64.size % row_len:
        raise ValueError("row_len must divide the element count")
    rows = x64.reshape(-1, row_len)
    amax = np.abs(rows).max(axis=1)
    e = pow2_exponent(amax)
    codes = e4m3_encode(rows * np.ldexp(1.0, -e)[:, None])
    return codes.reshape(np.shape(x)), (e + 127).astype(np.uint8)


def attention_fp8_rows(q8, k8, v8, q_e8m0, k_e8m0, s_v, scale, rows=None):
    """Attention on row-scaled E4M3 Q and K (one power-of-two scale per token,
    E8M0 bytes [B,H,N]) and per-tensor E4M3 V (scale s_v), with P quantised
    to E4M3 at x448 exactly as ``attention_fp8``."""
    q = e4m3_decode(np.asarray(q8)) * np.ldexp(1.0, np.asarray(q_e8m0, dtype=np.int64) - 127)[..., None]
    k = e4m3_decode(np.asarray(k8)) * np.ldexp(1.0, np.asarray(k_e8m0, dtype=np.int64) - 127)[..., None]
    v = e4m3_decode(np.asarray(v8)) * float(s_v)
    return _attention_p8(q, k, v, scale, rows)


def _attention_p8(q, k, v, scale, rows):
    """Softmax attention on dequantised float64 q, k, v with the
    probabilities rounded to E4M3 at x448 before the P.V product and the
    normaliser taken from the unrounded probabilities."""
    B, H, Nq, D = q.shape
    if k.shape[2] < 1:
        raise ValueError("Nkv must be >= 1")
    if rows is not None:
        q = q[:, :, np.asarray(rows, dtype=np.int64), :]
    nq = q.shape[2]
    o = np.empty((B, H, nq, D), dtype=np.float64)
    lse = np.empty((B, H, nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = float(scale) * (q[b, h] @ k[b, h].T)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            p8 = e4m3_round(E4M3_MAX * p)
            o[b, h] = (p8 @ v[b, h]) / (E4M3_MAX * l)
            lse[b, h] = m[:, 0] + np.log(l[:, 0])
    return o, lse


def p_block_ids(nkv, block):
    """Block label of each of ``nkv`` keys for per-block P scales: ``block``
    consecutive keys share a label, key j is in block j // block (the last
    block may be shorter). The pages leave the granularity of P's scale
    open, so the block size is a parameter of the definition."""
    block = int(block)
    if block < 1:
        raise ValueError("block must be >= 1")
    return np.arange(int(nkv)) // block


def p_block_exponents(pv, blocks):
    """One power-of-two exponent per (row, block) of the non-negative values
    pv [rows, Nkv]: e = pow2_exponent(the block's largest value), so that
    value lands in (224, 448] * 2^e (e = 0 for an all-zero block). ``blocks``
    labels the keys 0, 0, .., 1, 1, .. in runs (as ``p_block_ids`` does).
    Returns e of shape [rows, n_blocks]."""
    pv = np.asarray(pv, dtype=np.float64)
    blocks = np.asarray(blocks)
    starts = np.flatnonzero(np.r_[True, blocks[1:] != blocks[:-1]])
    if not np.array_equal(blocks[starts], np.arange(starts.size)):
        raise ValueError("blocks must label consecutive runs 0, 1, 2, ...")
    bmax = np.maximum.reduceat(pv, starts, axis=1)
    return pow2_exponent(bmax)


def quant_p_blocks(pv, blocks):
    """E4M3 codes of the probabilities pv [rows, Nkv] with one power-of-two
    scale per (row, block): 2^e with e from ``p_block_exponents``. Returns
    (codes, e) with e of shape [rows, n_blocks]."""
    pv = np.asarray(pv, dtype=np.float64)
    e = p_block_exponents(pv, blocks)
    codes = e4m3_encode(pv * np.ldexp(1.0, -e[:, np.asarray(blocks)]))
    return codes, e


def attention_fp8_rows_v(q8, k8, v8, q_e8m0, k_e8m0, v_e8m0, scale, *, block, rows=None):
    """Row-wise fp8 attention with per-token scales for Q, K and V and
    per-block scales for P (ParaAttention guide, section "fp8 quantization":
    row-wise scaling as the more accurate option).

    Q, K and V are E4M3 codes with one power-of-two scale per token (E8M0
    bytes [B,H,N]). With p = exp(s - m) as in ``attention_fp8``, V's scale is
    folded into the probabilities, pv_j = p_j * 2^(ev_j - 127), which are
    rounded to E4M3 with one power-of-two scale per (query, block of
    ``block`` consecutive keys; ``p_block_ids``) before the product with V's
    codes: O = sum_j P^_j * v8_j / sum_j p_j, LSE = m + ln sum_j p_j, where
    P^ is the dequantised pv. ``block`` is required: the pages do not fix the
    granularity (1 gives every key its own scale; Nkv or more one scale per
    query row). A block shares one scale, so inside a block pv values more
    than E4M3's span (about 2^17) below the block maximum round to zero; a
    per-tensor V scale has the same limit over the whole tensor.
    """
    q = e4m3_decode(np.asarray(q8)) * np.ldexp(1.0, np.asarray(q_e8m0, dtype=np.int64) - 127)[..., None]
    k = e4m3_decode(np.asarray(k8)) * np.ldexp(1.0, np.asarray(k_e8m0, dtype=np.int64) - 127)[..., None]
    vq = e4m3_decode(np.asarray(v8))
    ev = np.asarray(v_e8m0, dtype=np.int64) - 127
    B, H, Nq, D = q.shape
    nkv = k.shape[2]
    if nkv < 1:
        raise ValueError("Nkv must be >= 1")
    if rows is not None:
        q = q[:, :, np.asarray(rows, dtype=np.int64), :]
    nq = q.shape[2]
    blocks = p_block_ids(nkv, block)
    o = np.empty((B, H, nq, D), dtype=np.float64)
    lse = np.empty((B, H, nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = float(scale) * (q[b, h] @ k[b, h].T)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            pv = p * np.ldexp(1.0, ev[b, h])[None, :]
            f = np.ldexp(1.0, p_block_exponents(pv, blocks))[:, blocks]
            pq = e4m3_round(pv / f) * f
            o[b, h] = (pq @ vq[b, h]) / l
            lse[b, h] = m[:, 0] + np.log(l[:, 0])
    return o, lse
