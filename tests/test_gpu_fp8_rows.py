"""GPU parity of the row-wise fp8 variant: fp8_quant_rows_pow2 (bit-exact
codes and E8M0 exponents) and attn_fwd_fp8_rows (against the oracle on the
dequantised inputs and on the bf16 inputs), through the C ABI."""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
import oracle
import workloads
from helpers import (FP8_O_MEAN_ABS, FP8_REL_L2_VS_BF16, FP8_REL_L2_VS_DEQUANT,
                     KERNEL_P_BLOCK, KERNEL_P_SCALE, LSE_ABS, assert_bf16_attention,
                     assert_within_bound, deq_per_tensor, deq_rows, fp8_p_rounding_bound,
                     head_groups, rel_l2, take_rows, to64)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("rows,row_len", [(77, 128), (16, 64), (5, 8), (33, 136)])
def test_quant_rows_bit_exact(rows, row_len):
    print("CASE rows_pow2 %d x %d" % (rows, row_len), flush=True)
    g = torch.Generator().manual_seed(rows * 1000 + row_len)
    mag = torch.exp2(torch.randint(-30, 30, (rows, 1), generator=g).float())
    x = (torch.randn(rows, row_len, generator=g) * mag)
    x[0] = 0.0                                           # all-zero row -> exponent 0
    if rows > 3:
        x[1, 0] = 448.0 * 2.0 ** 5                       # amax exactly 448 * 2^5
        x[2, 0] = 448.0 * 2.0 ** -3 * (1 + 2.0 ** -7)    # just above a power
        x[3, :] = 1e-38                                  # tiny rows clamp at 2^-127
    x = x.to(torch.bfloat16)
    x8, e8 = dta.fp8_quant_rows_pow2(x.to(DEV), row_len)
    torch.cuda.synchronize()
    codes, e_ref = oracle.quant_rows_pow2(x, row_len)
    assert np.array_equal(e8.cpu().numpy().ravel(), e_ref)
    assert np.array_equal(x8.cpu().numpy(), codes)


def test_quant_rows_flux_q_bit_exact():
    print("CASE rows_pow2 flux Q", flush=True)
    q, _, _ = workloads.workload_qkv("flux_1024", device=DEV)
    q8, e8 = dta.fp8_quant_rows_pow2(q)
    torch.cuda.synchronize()
    codes, e_ref = oracle.quant_rows_pow2(q.cpu(), q.shape[-1])
    assert np.array_equal(e8.cpu().numpy().ravel(), e_ref)
    assert np.array_equal(q8.cpu().numpy(), codes)


def _rows_path(q, k, v):
    q8, eq = dta.fp8_quant_rows_pow2(q)
    k8, ek = dta.fp8_quant_rows_pow2(k)
    v8, sv = dta.fp8_quant_per_tensor(v)
    return q8, k8, v8, eq, ek, sv


def _gates(acc, what):
    a = {key: np.concatenate(val, axis=1) for key, val in acc.items()}
    o8, l8 = a["o"], a["l"]
    assert np.isfinite(o8).all() and np.isfinite(l8).all()
    mean_abs = np.abs(o8 - a["bf"]).mean()
    r_bf, r_dq = rel_l2(o8, a["bf"]), rel_l2(o8, a["dq"])
    e_l = np.abs(l8 - a["ldq"]).max()
    msg = "%s: O mean-abs %.3e, rel-L2 %.3e (bf16) %.3e (dequant), LSE %.3e" % (
        what, mean_abs, r_bf, r_dq, e_l)
    print(msg)
    assert mean_abs <= FP8_O_MEAN_ABS and r_bf <= FP8_REL_L2_VS_BF16, msg
    assert r_dq <= FP8_REL_L2_VS_DEQUANT and e_l <= LSE_ABS, msg
    assert_within_bound(o8, a["star"], a["bound"], what)
    return r_bf


def _check(o8, l8, q, k, v, q8, k8, v8, eq, ek, sv, scale, rows=None, what=""):
    """Gates and the elementwise P-rounding bound (x108 P, as attn_fwd_fp8);
    rows None: every row, else [H, r] rows per head."""
    q8n, k8n, v8n, eqn, ekn = (t.cpu().numpy() for t in (q8, k8, v8, eq, ek))
    s_v = float(sv.item())
    acc = {key: [] for key in ("o", "l", "bf", "dq", "ldq", "star", "bound")}
    for hs, r in head_groups(rows, q.shape[1]):
        o_dq, l_dq = oracle.attention_fp8_rows(q8n[:, hs], k8n[:, hs], v8n[:, hs], eqn[:, hs],
                                               ekn[:, hs], s_v, scale, rows=r)
        o_bf, _ = oracle.attention(q[:, hs].cpu(), k[:, hs].cpu(), v[:, hs].cpu(), scale, rows=r)
        o_st, bd = fp8_p_rounding_bound(deq_rows(q8n[:, hs], eqn[:, hs]),
                                        deq_rows(k8n[:, hs], ekn[:, hs]),
                                        deq_per_tensor(v8n[:, hs], s_v), scale,
                                        p_scale=KERNEL_P_SCALE, rows=r)
        for key, val in (("o", to64(take_rows(o8, hs, r))), ("l", to64(take_rows(l8, hs, r))),
                         ("bf", o_bf), ("dq", o_dq), ("ldq", l_dq), ("star", o_st),
                         ("bound", bd)):
            acc[key].append(val)
    return _gates(acc, what)


@pytest.mark.parametrize("B,H,Nq,Nkv,D", [(1, 2, 300, 300, 128), (1, 3, 200, 131, 64),
                                          (1, 1, 64, 1, 128), (2, 1, 97, 640, 128)])
def test_attention_rows_shapes(B, H, Nq, Nkv, D):
    print("CASE fp8 rows shape", B, H, Nq, Nkv, D, flush=True)
    q, k, v = workloads.make_qkv(23, B, H, Nq, Nkv, D, device=DEV)
    q8, k8, v8, eq, ek, sv = _rows_path(q, k, v)
    o8, l8 = dta.attn_fwd_fp8_rows(q8, k8, v8, eq, ek, sv, D ** -0.5)
    torch.cuda.synchronize()
    _check(o8, l8, q, k, v, q8, k8, v8, eq, ek, sv, D ** -0.5, what="fp8 rows")


def test_attention_rows_flux_rows_per_head():
    c = workloads.CONFIGS["flux_1024_fp8"]
    print("CASE fp8 rows flux", flush=True)
    q, k, v = workloads.workload_qkv("flux_1024_fp8", device=DEV)
    q8, k8, v8, eq, ek, sv = _rows_path(q, k, v)
    o8, l8 = dta.attn_fwd_fp8_rows(q8, k8, v8, eq, ek, sv, c["D"] ** -0.5)
    torch.cuda.synchronize()
    rows = workloads.sample_rows_per_head(c["config"], c["N"], c["H"], 256, c["n_text"])
    _check(o8, l8, q, k, v, q8, k8, v8, eq, ek, sv, c["D"] ** -0.5, rows=rows, what="fp8 rows flux")


def _video_length_inputs():
    # Two heads of the HunyuanVideo 720p x 129-frame recipe at its full
    # sequence length (119 056 tokens: 1861 K/V tiles, the last one 16 keys),
    # 256 rows per head (forced edge rows, one in each 32-row block dealt to
    # the head).
    c = workloads.CONFIGS["hunyuan_720p_129f"]
    N, D = c["N"], c["D"]
    q, k, v = workloads.make_qkv(c["config"], 1, 2, N, N, D, device=DEV)
    return q, k, v, D ** -0.5, workloads.sample_rows_per_head(c["config"], N, 2, 256, c["n_text"])


def test_attention_rows_video_length_rows_per_head():
    print("CASE fp8 rows video length, 2 heads", flush=True)
    q, k, v, scale, rows = _video_length_inputs()
    q8, k8, v8, eq, ek, sv = _rows_path(q, k, v)
    o8, l8 = dta.attn_fwd_fp8_rows(q8, k8, v8, eq, ek, sv, scale)
    torch.cuda.synchronize()
    _check(o8, l8, q, k, v, q8, k8, v8, eq, ek, sv, scale, rows=rows, what="fp8 rows video length")


def test_uniform_exponents_match_per_tensor_bitwise():
    """With every row exponent equal, the MFMA operand scales 2^(eq+ek) and
    the per-tensor path's float factor s_q s_k = 2^(eq+ek) give the same
    logits exactly, so both kernels must agree bit for bit."""
    B, H, N, D = 1, 2, 250, 128
    q, k, v = workloads.make_qkv(24, B, H, N, N, D, device=DEV)
    q8, _ = dta.fp8_quant_rows_pow2(q)
    k8, _ = dta.fp8_quant_rows_pow2(k)
    v8, sv = dta.fp8_quant_per_tensor(v)
    eq = torch.full((B, H, N), 127 - 3, dtype=torch.uint8, device=DEV)
    ek = torch.full((B, H, N), 127 + 2, dtype=torch.uint8, device=DEV)
    o_r, l_r = dta.attn_fwd_fp8_rows(q8, k8, v8, eq, ek, sv, D ** -0.5)
    ds = torch.cat([torch.tensor([2.0 ** -3, 2.0 ** 2], device=DEV), sv])
    o_t, l_t = dta.attn_fwd_fp8(q8, k8, v8, ds, D ** -0.5)
    torch.cuda.synchronize()
    assert torch.equal(o_r, o_t) and torch.equal(l_r, l_t)


def test_outlier_tokens_row_wise_beats_per_tensor():
    B, H, N, D = 1, 2, 256, 128
    q, k, v = workloads.make_qkv(25, B, H, N, N, D, device=DEV)
    q = q.float()
    q[:, :, 7] *= 65536.0
    q = q.to(torch.bfloat16)
    scale = D ** -0.5
    o_ref, _ = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    q8, k8, v8, eq, ek, sv = _rows_path(q, k, v)
    o_r, _ = dta.attn_fwd_fp8_rows(q8, k8, v8, eq, ek, sv, scale)
    qt, sq = dta.fp8_quant_per_tensor(q)
    kt, sk = dta.fp8_quant_per_tensor(k)
    o_t, _ = dta.attn_fwd_fp8(qt, kt, v8, torch.cat([sq, sk, sv]), scale)
    torch.cuda.synchronize()
    keep = [i for i in range(N) if i != 7]
    err_r = rel_l2(to64(o_r)[:, :, keep], o_ref[:, :, keep])
    err_t = rel_l2(to64(o_t)[:, :, keep], o_ref[:, :, keep])
    print("outlier token: rel-L2 row-wise %.3e, per-tensor %.3e" % (err_r, err_t))
    assert err_r <= FP8_REL_L2_VS_BF16 and err_t > 2 * err_r


# ---- per-token V and per-block P scales: attn_fwd_fp8_rows_v ----

def _rows_v_path(q, k, v):
    q8, eq = dta.fp8_quant_rows_pow2(q)
    k8, ek = dta.fp8_quant_rows_pow2(k)
    v8, ev = dta.fp8_quant_rows_pow2(v)
    return q8, k8, v8, eq, ek, ev


def _check_v(o8, l8, q, k, v, q8, k8, v8, eq, ek, ev, scale, rows=None, what=""):
    """Gates against the oracle with one P scale per (query, 32 consecutive
    keys) -- the block attn_fwd_fp8_rows_v documents -- and the per-block
    elementwise bound; rows None: every row, else [H, r] rows per head."""
    q8n, k8n, v8n, eqn, ekn, evn = (t.cpu().numpy() for t in (q8, k8, v8, eq, ek, ev))
    acc = {key: [] for key in ("o", "l", "bf", "dq", "ldq", "star", "bound")}
    for hs, r in head_groups(rows, q.shape[1]):
        o_dq, l_dq = oracle.attention_fp8_rows_v(q8n[:, hs], k8n[:, hs], v8n[:, hs], eqn[:, hs],
                                                 ekn[:, hs], evn[:, hs], scale,
                                                 block=KERNEL_P_BLOCK, rows=r)
        o_bf, _ = oracle.attention(q[:, hs].cpu(), k[:, hs].cpu(), v[:, hs].cpu(), scale, rows=r)
        ev_h = evn[:, hs].astype(np.int64).reshape(v8n[:, hs].shape[:-1]) - 127
        o_st, bd = fp8_p_rounding_bound(deq_rows(q8n[:, hs], eqn[:, hs]),
                                        deq_rows(k8n[:, hs], ekn[:, hs]),
                                        deq_rows(v8n[:, hs], evn[:, hs]), scale,
                                        vq=oracle.e4m3_decode(v8n[:, hs]), ev=ev_h,
                                        block=KERNEL_P_BLOCK, rows=r)
        for key, val in (("o", to64(take_rows(o8, hs, r))), ("l", to64(take_rows(l8, hs, r))),
                         ("bf", o_bf), ("dq", o_dq), ("ldq", l_dq), ("star", o_st),
                         ("bound", bd)):
            acc[key].append(val)
    return _gates(acc, what)


@pytest.mark.parametrize("B,H,Nq,Nkv,D", [(1, 2, 300, 300, 128), (1, 3, 200, 131, 64),
                                          (1, 1, 64, 1, 128), (2, 1, 97, 640, 128),
                                          (1, 2, 129, 65, 64)])
def test_attention_rows_v_shapes(B, H, Nq, Nkv, D):
    print("CASE fp8 rows_v shape", B, H, Nq, Nkv, D, flush=True)
    q, k, v = workloads.make_qkv(27, B, H, Nq, Nkv, D, device=DEV)
    q8, k8, v8, eq, ek, ev = _rows_v_path(q, k, v)
    o8, l8 = dta.attn_fwd_fp8_rows_v(q8, k8, v8, eq, ek, ev, D ** -0.5)
    torch.cuda.synchronize()
    _check_v(o8, l8, q, k, v, q8, k8, v8, eq, ek, ev, D ** -0.5, what="fp8 rows_v")


def test_attention_rows_v_flux_rows_per_head():
    c = workloads.CONFIGS["flux_1024_fp8"]
    print("CASE fp8 rows_v flux", flush=True)
    q, k, v = workloads.workload_qkv("flux_1024_fp8", device=DEV)
    q8, k8, v8, eq, ek, ev = _rows_v_path(q, k, v)
    o8, l8 = dta.attn_fwd_fp8_rows_v(q8, k8, v8, eq, ek, ev, c["D"] ** -0.5)
    torch.cuda.synchronize()
    rows = workloads.sample_rows_per_head(c["config"], c["N"], c["H"], 256, c["n_text"])
    _check_v(o8, l8, q, k, v, q8, k8, v8, eq, ek, ev, c["D"] ** -0.5, rows=rows,
             what="fp8 rows_v flux")


def test_attention_rows_v_video_length_rows_per_head():
    print("CASE fp8 rows_v video length, 2 heads", flush=True)
    q, k, v, scale, rows = _video_length_inputs()
    q8, k8, v8, eq, ek, ev = _rows_v_path(q, k, v)
    o8, l8 = dta.attn_fwd_fp8_rows_v(q8, k8, v8, eq, ek, ev, scale)
    torch.cuda.synchronize()
    _check_v(o8, l8, q, k, v, q8, k8, v8, eq, ek, ev, scale, rows=rows,
             what="fp8 rows_v video length")


def test_rows_v_uniform_scores_give_the_mean_of_v():
    """Q = 0: every p is 1 and every block's pv is a power of two that E4M3
    holds exactly, so O is the mean of the dequantised V rows (to float32
    accumulation and one bf16 rounding) and LSE = ln N."""
    B, H, N, D = 1, 2, 333, 128
    print("CASE fp8 rows_v uniform scores", flush=True)
    _, k, v = workloads.make_qkv(28, B, H, N, N, D, device=DEV)
    g = torch.Generator().manual_seed(5)
    v = (v.float() * torch.exp2(torch.randint(-6, 7, (B, H, N, 1), generator=g).float().to(DEV))
         ).to(torch.bfloat16)
    q = torch.zeros(B, H, N, D, dtype=torch.bfloat16, device=DEV)
    q8, k8, v8, eq, ek, ev = _rows_v_path(q, k, v)
    o8, l8 = dta.attn_fwd_fp8_rows_v(q8, k8, v8, eq, ek, ev, D ** -0.5)
    torch.cuda.synchronize()
    v_deq = oracle.e4m3_decode(v8.cpu().numpy()) * np.exp2(
        ev.cpu().numpy().reshape(B, H, N, 1).astype(np.float64) - 127)
    mean = np.broadcast_to(v_deq.mean(axis=2, keepdims=True), (B, H, N, D))
    o = to64(o8)
    ulp = np.maximum(np.abs(mean), 2.0 ** -126) * 2.0 ** -8
    assert (np.abs(o - mean) <= ulp + 1e-5 * np.abs(v_deq).max()).all()
    assert np.abs(to64(l8) - np.log(N)).max() < 1e-5


def test_rows_v_outlier_value_token_beats_per_tensor_v():
    B, H, N, D = 1, 2, 256, 128
    print("CASE fp8 rows_v outlier V token", flush=True)
    q, k, v = workloads.make_qkv(29, B, H, N, N, D, device=DEV)
    v = v.float()
    v[:, :, 7, :8] *= 65536.0
    v[:, :, 7, 8:] = 0.0
    v = v.to(torch.bfloat16)
    scale = D ** -0.5
    o_ref, _ = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    q8, k8, v8, eq, ek, ev = _rows_v_path(q, k, v)
    o_v, _ = dta.attn_fwd_fp8_rows_v(q8, k8, v8, eq, ek, ev, scale)
    vt, sv = dta.fp8_quant_per_tensor(v)
    o_t, _ = dta.attn_fwd_fp8_rows(q8, k8, vt, eq, ek, sv, scale)
    torch.cuda.synchronize()
    d = slice(8, None)
    err_v = rel_l2(to64(o_v)[..., d], o_ref[..., d])
    err_t = rel_l2(to64(o_t)[..., d], o_ref[..., d])
    print("outlier V token: rel-L2 per-token V %.3e, per-tensor V %.3e" % (err_v, err_t))
    assert err_v <= FP8_REL_L2_VS_BF16 and err_t > 1.6 * err_v


def test_rows_v_keeps_a_diffuse_tail():
    """One query over 60000 keys: a peak and a tail at p ~ 1e-6 per key. The
    x108 P scaling of attn_fwd_fp8_rows rounds the tail to zero; the
    per-block P scales keep it (reference: exact attention on the
    dequantised inputs)."""
    N, D = 60000, 64
    print("CASE fp8 rows_v diffuse tail", flush=True)
    g = torch.Generator().manual_seed(30)
    q = torch.zeros(1, 1, 1, D)
    q[..., 0] = 4.0
    k = torch.zeros(1, 1, N, D)
    k[0, 0, 1:, 0] = -torch.log(torch.tensor(1e6)) / 4.0 * (1.0 + 0.01 * torch.randn(N - 1, generator=g))
    v = 1.0 + torch.rand(1, 1, N, D, generator=g)
    v[0, 0, 0] = 0.0
    q, k, v = (t.to(torch.bfloat16).to(DEV) for t in (q, k, v))
    q8, k8, v8, eq, ek, ev = _rows_v_path(q, k, v)
    o_v, l_v = dta.attn_fwd_fp8_rows_v(q8, k8, v8, eq, ek, ev, 1.0)
    vt, sv = dta.fp8_quant_per_tensor(v)
    o_t, _ = dta.attn_fwd_fp8_rows(q8, k8, vt, eq, ek, sv, 1.0)
    torch.cuda.synchronize()
    deq = [oracle.e4m3_decode(c.cpu().numpy()) *
           np.exp2(e.cpu().numpy().reshape(sh + (1,)).astype(np.float64) - 127)
           for c, e, sh in ((q8, eq, (1, 1, 1)), (k8, ek, (1, 1, N)), (v8, ev, (1, 1, N)))]
    o_ref, l_ref = oracle.attention(*deq, 1.0)
    err_v = rel_l2(to64(o_v), o_ref)
    err_t = rel_l2(to64(o_t), o_ref)
    print("diffuse tail: rel-L2 per-block P %.3e, x108 P %.3e" % (err_v, err_t))
    assert err_v < 0.02 and err_t > 0.9
    assert np.abs(to64(l_v) - l_ref).max() < LSE_ABS


@pytest.mark.parametrize("Nkv", [40, 128, 150, 192, 385])
def test_attention_rows_tile_counts(Nkv):
    """Tile counts 1 to 7 with full and ragged last tiles for the skewed
    8-wave instance (three LDS buffers, the skewed waves' last P.V after the
    loop)."""
    print("CASE fp8 rows tile count", Nkv, flush=True)
    q, k, v = workloads.make_qkv(29, 1, 2, 300, Nkv, 128, device=DEV)
    q8, k8, v8, eq, ek, sv = _rows_path(q, k, v)
    o8, l8 = dta.attn_fwd_fp8_rows(q8, k8, v8, eq, ek, sv, 128 ** -0.5)
    torch.cuda.synchronize()
    _check(o8, l8, q, k, v, q8, k8, v8, eq, ek, sv, 128 ** -0.5, what="rows Nkv=%d" % Nkv)


def test_rows_query_position_invariance():
    """Rolling the queries (and their exponents) by 128 rows moves them between
    the on-time and the skewed waves of a workgroup; O and LSE roll bit for
    bit."""
    print("CASE fp8 rows query roll", flush=True)
    q, k, v = workloads.make_qkv(31, 1, 2, 512, 300, 128, device=DEV)
    q8, k8, v8, eq, ek, sv = _rows_path(q, k, v)
    o_a, l_a = dta.attn_fwd_fp8_rows(q8, k8, v8, eq, ek, sv, 128 ** -0.5)
    o_b, l_b = dta.attn_fwd_fp8_rows(torch.roll(q8, 128, dims=2).contiguous(), k8, v8,
                                     torch.roll(eq, 128, dims=2).contiguous(), ek, sv,
                                     128 ** -0.5)
    torch.cuda.synchronize()
    assert torch.equal(torch.roll(o_a, 128, dims=2), o_b)
    assert torch.equal(torch.roll(l_a, 128, dims=2), l_b)
