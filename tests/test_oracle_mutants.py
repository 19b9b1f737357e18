"""The oracle's pins catch plausible mistakes (no GPU).

Each mutant below plants one slip in an oracle function, the kind of slip
the pins in test_oracle_pins.py are there to catch: a dropped or doubled
scale, a wrong logarithm base, a dropped max term, a missing normalisation,
a softmax over the wrong axis, an off-by-one key, a wrong sign, the wrong
merge weights, a wrong residual denominator, wrong E4M3 rounding, bias,
saturation or subnormals. With the mutant patched into ``oracle`` (on the
CPU only), at least one of the pins that cover that function must fail; with
the real oracle every one of them passes.
"""

import importlib
import math

import numpy as np
import pytest

import oracle
import oracle.fp8 as ofp8
import test_fp8_bound as fp8_bound
import test_oracle_pins as pins

ATTN, MERGE, RESID = oracle.attention, oracle.merge, oracle.residual_diff
ENC, DEC, RND = oracle.e4m3_encode, oracle.e4m3_decode, oracle.e4m3_round


def _f64(x):
    """float64 numpy copy of a numpy array or a torch tensor (any dtype)."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _logits(q, k, scale, rows):
    q, k = _f64(q), _f64(k)
    if rows is not None:
        q = q[:, :, np.asarray(rows)]
    return float(scale) * (q @ np.swapaxes(k, -1, -2))


def _row_max(q, k, scale, rows):
    return _logits(q, k, scale, rows).max(axis=-1)


# ---- attention ------------------------------------------------------------

def a_scale_dropped(q, k, v, scale, rows=None):
    return ATTN(q, k, v, 1.0, rows)


def a_scale_squared(q, k, v, scale, rows=None):
    return ATTN(q, k, v, float(scale) ** 2, rows)


def a_lse_log2(q, k, v, scale, rows=None):
    o, lse = ATTN(q, k, v, scale, rows)
    return o, lse / math.log(2.0)


def a_lse_without_max(q, k, v, scale, rows=None):
    o, lse = ATTN(q, k, v, scale, rows)
    return o, lse - _row_max(q, k, scale, rows)


def a_unnormalised(q, k, v, scale, rows=None):
    o, lse = ATTN(q, k, v, scale, rows)
    l = np.exp(lse - _row_max(q, k, scale, rows))
    return o * l[..., None], lse


def a_softmax_over_queries(q, k, v, scale, rows=None):
    s = _logits(q, k, scale, rows)
    m = s.max(axis=-2, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=-2, keepdims=True)
    o = p @ _f64(v)
    return o, (m + np.log(e.sum(axis=-2, keepdims=True)))[..., 0, :1].repeat(s.shape[-2], -1)


def a_last_key_dropped(q, k, v, scale, rows=None):
    k, v = _f64(k), _f64(v)
    if k.shape[2] > 1:
        k, v = k[:, :, :-1], v[:, :, :-1]
    return ATTN(q, k, v, scale, rows)


def a_values_off_by_one(q, k, v, scale, rows=None):
    return ATTN(q, k, np.roll(_f64(v), 1, axis=2), scale, rows)


def a_query_sign(q, k, v, scale, rows=None):
    return ATTN(-_f64(q), k, v, scale, rows)


def a_rows_ignored(q, k, v, scale, rows=None):
    return ATTN(q, k, v, scale)


# ---- merge ----------------------------------------------------------------

def _w(lse_parts, sign=1.0):
    lp = _f64(lse_parts)
    m = np.where(np.isfinite(lp.max(0)), lp.max(0), 0.0)
    with np.errstate(invalid="ignore", over="ignore"):
        return np.where(np.isneginf(lp), 0.0, np.exp(sign * (lp - m)))


def m_lse_is_max(o_parts, lse_parts):
    o, _ = MERGE(o_parts, lse_parts)
    return o, _f64(lse_parts).max(axis=0)


def m_equal_weights(o_parts, lse_parts):
    _, lse = MERGE(o_parts, lse_parts)
    return _f64(o_parts).mean(axis=0), lse


def m_weight_sign(o_parts, lse_parts):
    w = _w(lse_parts, -1.0)
    o = (w[..., None] * _f64(o_parts)).sum(0) / w.sum(0)[..., None]
    return o, MERGE(o_parts, lse_parts)[1]


def m_last_partial_dropped(o_parts, lse_parts):
    if np.shape(o_parts)[0] > 1:
        return MERGE(_f64(o_parts)[:-1], _f64(lse_parts)[:-1])
    return MERGE(o_parts, lse_parts)


def m_lse_log2(o_parts, lse_parts):
    o, lse = MERGE(o_parts, lse_parts)
    return o, lse / math.log(2.0)


# ---- residual_diff --------------------------------------------------------

def _f(x):
    return _f64(x).ravel()


def r_denominator_a(a, b):
    a, b = _f(a), _f(b)
    with np.errstate(divide="ignore", invalid="ignore"):
        return float(np.abs(a - b).sum() / np.abs(a).sum())


def r_no_abs(a, b):
    a, b = _f(a), _f(b)
    with np.errstate(divide="ignore", invalid="ignore"):
        return float(abs((a - b).sum()) / np.abs(b).sum())


def r_squared(a, b):
    a, b = _f(a), _f(b)
    with np.errstate(divide="ignore", invalid="ignore"):
        return float(((a - b) ** 2).sum() / (b ** 2).sum())


def r_swapped(a, b):
    return RESID(b, a)


# ---- E4M3 -----------------------------------------------------------------

def e_ties_away(x):
    return ENC(np.asarray(x, dtype=np.float64) * (1.0 + 2.0 ** -40))


def e_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    c = ENC(x).astype(np.int64)
    over = (np.abs(DEC(c)) > np.abs(x)) & ((c & 0x7F) > 0) & ~np.isnan(x)
    return np.where(over, c - 1, c).astype(np.uint8)


def e_no_saturation(x):
    x = np.asarray(x, dtype=np.float64)
    c = ENC(x)
    return np.where(np.abs(x) >= 464.0, np.uint8(0x7F), c).astype(np.uint8)


def e_flush_subnormals(x):
    c = ENC(x)
    return np.where((c & 0x7F) < 0x08, c & 0x80, c).astype(np.uint8)


def e_sign_lost(x):
    return ENC(np.abs(np.asarray(x, dtype=np.float64)))


def e_bias_8(x):
    return ENC(np.asarray(x, dtype=np.float64) * 2.0)


def d_bias_8(codes):
    return DEC(codes) / 2.0


def d_subnormal_as_normal(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sub = ((c >> 3) & 0xF) == 0
    m = (c & 0x7).astype(np.float64)
    bad = np.where(c & 0x80, -1.0, 1.0) * (1.0 + m / 8.0) * 2.0 ** -7
    return np.where(sub & ((c & 0x7) != 0), bad, DEC(codes))


def d_nan_is_480(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, np.where(c & 0x80, -480.0, 480.0), DEC(codes))


def q_ties_away(x):
    return RND(np.asarray(x, dtype=np.float64) * (1.0 + 2.0 ** -40))


def q_no_saturation(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(np.abs(x) > 448.0, x, RND(x))


def q_coarse_subnormals(x):
    x = np.asarray(x, dtype=np.float64)
    sub = np.abs(x) < 2.0 ** -6
    return np.where(sub, np.round(x / 2.0 ** -8) * 2.0 ** -8, RND(x))


# ---- layout ---------------------------------------------------------------

SEQ_SPLIT, SEQ_CONCAT = oracle.layout.seq_split, oracle.layout.seq_concat
HEAD_SPLIT, HEAD_CONCAT = oracle.layout.head_split, oracle.layout.head_concat


def l_split_one_late(x, lens, padded=None):
    x = np.asarray(x)
    return SEQ_SPLIT(np.roll(x, -1, axis=2), lens, padded)


def l_concat_reversed(parts, lens):
    return SEQ_CONCAT(list(parts)[::-1], list(lens)[::-1])


def l_padding_not_zero(x, lens, padded=None):
    out = SEQ_SPLIT(x, lens, padded)
    for part, n in zip(out, lens):
        part[:, :, n:] = 1
    return out


def l_head_cuts_off_by_one(x, heads):
    heads = list(heads)
    if len(heads) > 1 and heads[0] > 1:
        heads = [heads[0] - 1] + heads[1:-1] + [heads[-1] + 1]
    return HEAD_SPLIT(x, heads)


def l_head_concat_reversed(parts):
    return HEAD_CONCAT(list(parts)[::-1])


# ---- FBCache step -----------------------------------------------------------

FBC = oracle.fbcache_step


def f_not_strict(r, r_prev, threshold, hidden, cached):
    diff, use, out = FBC(r, r_prev, threshold, hidden, cached)
    if np.float32(diff) == np.float32(threshold):
        use = True
        out = FBC(r, r_prev, np.inf, hidden, cached)[2]
    return diff, use, out


def f_decided_in_float64(r, r_prev, threshold, hidden, cached):
    diff, _, _ = FBC(r, r_prev, threshold, hidden, cached)
    use = bool(diff < threshold)
    return diff, use, FBC(r, r_prev, np.inf if use else -np.inf, hidden, cached)[2]


def f_nan_reuses(r, r_prev, threshold, hidden, cached):
    diff, use, out = FBC(r, r_prev, threshold, hidden, cached)
    if np.isnan(diff):
        use = True
        out = FBC(r, r_prev, np.inf, hidden, cached)[2]
    return diff, use, out


def f_sum_not_rounded(r, r_prev, threshold, hidden, cached):
    diff, use, out = FBC(r, r_prev, threshold, hidden, cached)
    if use:
        out = _f64(hidden).reshape(np.shape(out)) + _f64(cached).reshape(np.shape(out))
    return diff, use, out


def b_truncates(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.where(np.isfinite(x), np.ldexp(np.trunc(m * 256.0) / 256.0, e), x)


# ---- row-wise fp8 -----------------------------------------------------------

POW2, PBLOCK = oracle.pow2_exponent, oracle.p_block_exponents


def p_exponent_one_high(amax):
    e = POW2(amax)
    return np.where(np.asarray(amax) == 0, e, e + 1)


def p_exponent_boundary(amax):
    amax = np.asarray(amax, dtype=np.float64)
    m, k = np.frexp(amax)
    e = np.where(m < 0.875, k - 9, k - 8)
    return np.where(amax == 0, 0, np.clip(e, -127, 127)).astype(np.int64)


def p_blocks_share_the_row_max(pv, blocks):
    e = PBLOCK(pv, blocks)
    return np.broadcast_to(e.max(axis=1, keepdims=True), e.shape).copy()


def p_blocks_take_the_min(pv, blocks):
    pv = np.asarray(pv, dtype=np.float64)
    blocks = np.asarray(blocks)
    starts = np.flatnonzero(np.r_[True, blocks[1:] != blocks[:-1]])
    return POW2(np.minimum.reduceat(pv, starts, axis=1))


# ---- per-tensor fp8 attention ------------------------------------------------

def _p8_attention(q8, k8, v8, descale, scale, rows=None, *, quantise=True,
                  norm_from_p8=False, lse_from_p8=False, shift=True, v_descale=True):
    """oracle.attention_fp8 rewritten with switches for the planted slips."""
    q = DEC(q8) * float(descale[0])
    k = DEC(k8) * float(descale[1])
    v = DEC(v8) * (float(descale[2]) if v_descale else 1.0)
    if rows is not None:
        q = q[:, :, np.asarray(rows)]
    s = float(scale) * (q @ np.swapaxes(k, -1, -2))
    m = s.max(axis=-1, keepdims=True) if shift else np.zeros_like(s[..., :1])
    p = np.exp(s - m)
    p8 = RND(448.0 * p) if quantise else 448.0 * p
    l = (p8 / 448.0 if norm_from_p8 else p).sum(axis=-1, keepdims=True)
    o = (p8 @ v) / (448.0 * l)
    lse_l = (p8 / 448.0 if lse_from_p8 else p).sum(axis=-1)
    return o, m[..., 0] + np.log(lse_l)


def g_p_not_quantised(*a, **kw):
    return _p8_attention(*a, quantise=False, **kw)


def g_normaliser_from_rounded_p(*a, **kw):
    return _p8_attention(*a, norm_from_p8=True, **kw)


def g_lse_from_rounded_p(*a, **kw):
    return _p8_attention(*a, lse_from_p8=True, **kw)


def g_no_max_shift(*a, **kw):
    return _p8_attention(*a, shift=False, **kw)


def g_v_descale_dropped(*a, **kw):
    return _p8_attention(*a, v_descale=False, **kw)


# ---- which pins cover which function ---------------------------------------

ATTN_PINS = [
    lambda: pins.test_z1_bruteforce_attention(3, 8, 4),
    pins.test_z1_bruteforce_merge_and_rows,
    pins.test_z2_softmax_rows_sum_to_one_and_identity_v,
    pins.test_z3_identical_keys_give_mean_v,
    pins.test_z4_constant_v,
    pins.test_z5_single_key,
    lambda: pins.test_z6_uniform_attention(True),
    lambda: pins.test_z6_uniform_attention(False),
    pins.test_z7_shift_of_all_keys,
    pins.test_z8_permutations,
    pins.test_z9_affine_in_v,
    pins.test_transposed_operand_is_caught,
    pins.test_z10_tiny_config_four_chunks,
    lambda: pins.test_z10_random_partitions(0),
    pins.test_z11_workload_statistics,
]
MERGE_PINS = [
    pins.test_z1_bruteforce_merge_and_rows,
    pins.test_z10_tiny_config_four_chunks,
    lambda: pins.test_z10_random_partitions(0),
    pins.test_merge_neg_inf_partials,
    pins.test_merge_single_partial_is_identity,
]
RESID_PINS = [
    pins.test_z1_bruteforce_residual_diff,
    pins.test_z12_residual_closed_forms,
    pins.test_z12_residual_workload_value,
]
FP8_PINS = [
    pins.test_z13_decode_all_codes_match_torch,
    pins.test_z13_encode_matches_torch_in_range,
    pins.test_z13_round_equals_encode_then_decode,
    pins.test_z13_encode_saturates,
    pins.test_z13_quant_per_tensor,
    pins.test_fp8_attention_identical_keys_exact,
    pins.test_fp8_attention_exact_power_of_two_probabilities,
]

LAYOUT_PINS = [
    pins.test_layout_seq_split_positions_by_formula,
    pins.test_layout_head_split_positions_by_formula,
    pins.test_layout_ulysses_round_trip_matches_global_slicing,
    pins.test_layout_ring_anything_pad_gather_trim,
]
FBCACHE_PINS = [
    pins.test_fbcache_bf16_round_matches_torch_from_float32,
    pins.test_fbcache_sum_is_correctly_rounded,
    pins.test_fbcache_decision_closed_forms,
    pins.test_fbcache_apply_rounds_the_sum_once_to_bf16,
    pins.test_fbcache_decision_is_taken_in_float32,
]
ROWS_PINS = [
    pins.test_rows_pow2_exponent_is_minimal,
    pins.test_rows_pow2_codes_match_torch_and_error_bound,
    pins.test_rows_pow2_attention_beats_per_tensor_on_outlier_tokens,
    lambda: pins.test_p_block_partition(32),
    pins.test_p_block_exponent_is_minimal_and_codes_match_torch,
    pins.test_rows_v_uniform_scores_give_the_mean_of_v,
    pins.test_rows_v_beats_per_tensor_v_on_an_outlier_value_token,
    pins.test_rows_v_keeps_a_diffuse_tail_that_x448_p_scaling_flushes,
    pins.test_rows_v_block_size_closed_form_uniform_scores,
    lambda: pins.test_rows_v_exact_power_of_two_probabilities(1),
    lambda: pins.test_rows_v_exact_power_of_two_probabilities(64),
]

FP8_ATTN_PINS = [
    pins.test_fp8_attention_identical_keys_exact,
    pins.test_fp8_attention_normalises_by_the_unrounded_probabilities,
    pins.test_fp8_attention_exact_power_of_two_probabilities,
    pins.test_fp8_attention_close_to_dequantised_attention,
    lambda: fp8_bound.test_oracle_x448_rounding_is_within_its_bound(1.0),
    lambda: fp8_bound.test_oracle_x448_rounding_is_within_its_bound(4.0),
]

# (name patched in ``oracle`` -- or in ``oracle.layout`` / ``oracle.residual``
# for a dotted name -- and, where the oracle calls it internally, in
# ``oracle.fp8``; the mutant; the pins that cover it)
MUTANTS = {
    "attention: scale dropped": ("attention", a_scale_dropped, ATTN_PINS),
    "attention: scale squared": ("attention", a_scale_squared, ATTN_PINS),
    "attention: LSE in log2": ("attention", a_lse_log2, ATTN_PINS),
    "attention: LSE without the row max": ("attention", a_lse_without_max, ATTN_PINS),
    "attention: O not divided by the row sum": ("attention", a_unnormalised, ATTN_PINS),
    "attention: softmax over queries": ("attention", a_softmax_over_queries, ATTN_PINS),
    "attention: last key dropped": ("attention", a_last_key_dropped, ATTN_PINS),
    "attention: values off by one key": ("attention", a_values_off_by_one, ATTN_PINS),
    "attention: query sign flipped": ("attention", a_query_sign, ATTN_PINS),
    "attention: rows argument ignored": ("attention", a_rows_ignored, ATTN_PINS),
    "merge: LSE is the max": ("merge", m_lse_is_max, MERGE_PINS),
    "merge: equal weights": ("merge", m_equal_weights, MERGE_PINS),
    "merge: weight exponent sign": ("merge", m_weight_sign, MERGE_PINS),
    "merge: last partial dropped": ("merge", m_last_partial_dropped, MERGE_PINS),
    "merge: LSE in log2": ("merge", m_lse_log2, MERGE_PINS),
    "residual: denominator |a|": ("residual_diff", r_denominator_a, RESID_PINS),
    "residual: no abs on the difference": ("residual_diff", r_no_abs, RESID_PINS),
    "residual: squared error": ("residual_diff", r_squared, RESID_PINS),
    "residual: arguments swapped": ("residual_diff", r_swapped, RESID_PINS),
    "e4m3 encode: ties away from zero": ("e4m3_encode", e_ties_away, FP8_PINS),
    "e4m3 encode: truncation": ("e4m3_encode", e_truncate, FP8_PINS),
    "e4m3 encode: no saturation": ("e4m3_encode", e_no_saturation, FP8_PINS),
    "e4m3 encode: subnormals flushed": ("e4m3_encode", e_flush_subnormals, FP8_PINS),
    "e4m3 encode: sign lost": ("e4m3_encode", e_sign_lost, FP8_PINS),
    "e4m3 encode: exponent bias 8": ("e4m3_encode", e_bias_8, FP8_PINS),
    "e4m3 decode: exponent bias 8": ("e4m3_decode", d_bias_8, FP8_PINS),
    "e4m3 decode: subnormals as normals": ("e4m3_decode", d_subnormal_as_normal, FP8_PINS),
    "e4m3 decode: NaN read as 480": ("e4m3_decode", d_nan_is_480, FP8_PINS),
    "e4m3 round: ties away from zero": ("e4m3_round", q_ties_away, FP8_PINS),
    "e4m3 round: no saturation": ("e4m3_round", q_no_saturation, FP8_PINS),
    "e4m3 round: subnormal spacing 2^-8": ("e4m3_round", q_coarse_subnormals, FP8_PINS),
    "layout: split parts one token late": ("layout.seq_split", l_split_one_late, LAYOUT_PINS),
    "layout: concat in reverse part order": ("layout.seq_concat", l_concat_reversed,
                                             LAYOUT_PINS),
    "layout: padding rows not zero": ("layout.seq_split", l_padding_not_zero, LAYOUT_PINS),
    "layout: head cuts off by one": ("layout.head_split", l_head_cuts_off_by_one, LAYOUT_PINS),
    "layout: head concat in reverse part order": ("layout.head_concat", l_head_concat_reversed,
                                                  LAYOUT_PINS),
    "fbcache: reuse at diff == threshold": ("fbcache_step", f_not_strict, FBCACHE_PINS),
    "fbcache: decision in float64": ("fbcache_step", f_decided_in_float64, FBCACHE_PINS),
    "fbcache: NaN diff reuses": ("fbcache_step", f_nan_reuses, FBCACHE_PINS),
    "fbcache: sum not rounded to bf16": ("fbcache_step", f_sum_not_rounded, FBCACHE_PINS),
    "fbcache: bf16 rounding truncates": ("residual._bf16_round", b_truncates, FBCACHE_PINS),
    "rows: exponent one too high": ("pow2_exponent", p_exponent_one_high, ROWS_PINS),
    "rows: exponent boundary at 448 exclusive": ("pow2_exponent", p_exponent_boundary,
                                                 ROWS_PINS),
    "rows: P blocks share the row maximum": ("p_block_exponents", p_blocks_share_the_row_max,
                                             ROWS_PINS),
    "rows: P block exponent from the block minimum": ("p_block_exponents",
                                                      p_blocks_take_the_min, ROWS_PINS),
    "fp8 attention: P not quantised": ("attention_fp8", g_p_not_quantised, FP8_ATTN_PINS),
    "fp8 attention: normaliser from the rounded P": ("attention_fp8",
                                                     g_normaliser_from_rounded_p, FP8_ATTN_PINS),
    "fp8 attention: LSE from the rounded P": ("attention_fp8", g_lse_from_rounded_p,
                                              FP8_ATTN_PINS),
    "fp8 attention: no max shift before rounding": ("attention_fp8", g_no_max_shift,
                                                    FP8_ATTN_PINS),
    "fp8 attention: V descale dropped": ("attention_fp8", g_v_descale_dropped, FP8_ATTN_PINS),
}


def _failures(pin_list):
    """Pins of the list whose assertions fail (any other exception would be
    a fault of the mutant or the harness, not a pin catching the slip, so it
    propagates)."""
    failed = 0
    for pin in pin_list:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            failed += 1
    return failed


def _patch(monkeypatch, name, fn):
    if "." in name:
        mod, attr = name.split(".")
        monkeypatch.setattr(getattr(oracle, mod) if mod == "layout" else
                            importlib.import_module("oracle." + mod), attr, fn)
        return
    monkeypatch.setattr(oracle, name, fn)
    if hasattr(ofp8, name):
        monkeypatch.setattr(ofp8, name, fn)


@pytest.mark.parametrize("pin_list", [ATTN_PINS, MERGE_PINS, RESID_PINS, FP8_PINS, LAYOUT_PINS,
                                      FBCACHE_PINS, ROWS_PINS, FP8_ATTN_PINS],
                         ids=["attention", "merge", "residual", "fp8", "layout", "fbcache",
                              "rows", "fp8 attention"])
def test_pins_pass_on_the_real_oracle(pin_list):
    assert _failures(pin_list) == 0


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_a_planted_mistake_fails_a_pin(mutant, monkeypatch):
    name, fn, pin_list = MUTANTS[mutant]
    _patch(monkeypatch, name, fn)
    assert _failures(pin_list) > 0, "no pin catches: " + mutant
