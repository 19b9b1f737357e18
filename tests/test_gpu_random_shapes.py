"""Seeded random shapes through every attention entry point, against the
oracle: bf16 attention, the fused ring step over random chunkings, and the
three fp8 variants. The shapes are drawn once from a fixed seed, so the cases
are the same on every run; each prints its shape before it runs."""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
import oracle
import workloads
from helpers import (FP8_O_MEAN_ABS, FP8_REL_L2_VS_BF16, FP8_REL_L2_VS_DEQUANT,
                     KERNEL_P_BLOCK, KERNEL_P_SCALE, LSE_ABS, assert_bf16_attention,
                     assert_within_bound, deq_per_tensor, deq_rows, fp8_p_rounding_bound,
                     rel_l2, to64)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _shapes(n, seed=20261203, hi=600):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        Nq = int(rng.integers(1, hi))
        Nkv = int(rng.integers(1, hi))
        D = int(rng.choice([64, 128]))
        out.append((B, H, Nq, Nkv, D))
    return out


# 8 short shapes, then 16 up to 2000 rows: several query tiles per head and
# K/V loops of up to 32 tiles, each with its own ragged tails.
SHAPES = _shapes(8) + _shapes(16, seed=20261204, hi=2000)


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_random_shape_bf16_and_ring(i):
    B, H, Nq, Nkv, D = SHAPES[i]
    print("CASE random bf16 + ring", SHAPES[i], flush=True)
    q, k, v = workloads.make_qkv(100 + i, B, H, Nq, Nkv, D, device=DEV)
    scale = D ** -0.5
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    o, lse = dta.attn_fwd(q, k, v, scale)
    torch.cuda.synchronize()
    assert_bf16_attention(o, lse, o_ref, lse_ref, "random bf16 %s" % (SHAPES[i],))
    # The same attention as a ring over a random chunking of the keys.
    rng = np.random.default_rng(200 + i)
    n_chunks = int(rng.integers(1, min(Nkv, 5) + 1))
    cuts = np.sort(rng.choice(np.arange(1, Nkv), size=n_chunks - 1, replace=False)) \
        if n_chunks > 1 else np.array([], dtype=np.int64)
    lens = np.diff(np.concatenate([[0], cuts, [Nkv]])).astype(int).tolist()
    print("  chunks", lens, flush=True)
    chunks = workloads.split_kv(k, v, lens)
    o_r, lse_r = dta.attn_fwd(q, chunks[0][0], chunks[0][1], scale)
    for kc, vc in chunks[1:]:
        dta.attn_fwd_accum(q, kc, vc, o_r, lse_r, scale)
    torch.cuda.synchronize()
    assert_bf16_attention(o_r, lse_r, o_ref, lse_ref, "random ring %s" % (lens,))


def _gates(o8, l8, o_bf, o_dq, l_dq, what):
    o8, l8 = to64(o8), to64(l8)
    assert np.isfinite(o8).all() and np.isfinite(l8).all(), what
    mean_abs = np.abs(o8 - o_bf).mean()
    r_bf, r_dq = rel_l2(o8, o_bf), rel_l2(o8, o_dq)
    e_l = np.abs(l8 - l_dq).max()
    msg = "%s: O mean-abs %.3e, rel-L2 %.3e (bf16) %.3e (dequant), LSE %.3e" % (
        what, mean_abs, r_bf, r_dq, e_l)
    print(msg)
    assert mean_abs <= FP8_O_MEAN_ABS and r_bf <= FP8_REL_L2_VS_BF16, msg
    assert r_dq <= FP8_REL_L2_VS_DEQUANT and e_l <= LSE_ABS, msg


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_random_shape_fp8_variants(i):
    B, H, Nq, Nkv, D = SHAPES[i]
    print("CASE random fp8", SHAPES[i], flush=True)
    q, k, v = workloads.make_qkv(300 + i, B, H, Nq, Nkv, D, device=DEV)
    scale = D ** -0.5
    o_bf, _ = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    # per tensor
    q8, sq = dta.fp8_quant_per_tensor(q)
    k8, sk = dta.fp8_quant_per_tensor(k)
    v8, sv = dta.fp8_quant_per_tensor(v)
    ds = torch.cat([sq, sk, sv])
    o8, l8 = dta.attn_fwd_fp8(q8, k8, v8, ds, scale)
    torch.cuda.synchronize()
    o_dq, l_dq = oracle.attention_fp8(q8.cpu().numpy(), k8.cpu().numpy(), v8.cpu().numpy(),
                                      ds.cpu().tolist(), scale)
    _gates(o8, l8, o_bf, o_dq, l_dq, "random fp8 per-tensor")
    dsc = ds.cpu().tolist()
    o_st, bd = fp8_p_rounding_bound(deq_per_tensor(q8, dsc[0]), deq_per_tensor(k8, dsc[1]),
                                    deq_per_tensor(v8, dsc[2]), scale, p_scale=KERNEL_P_SCALE)
    assert_within_bound(o8, o_st, bd, "random fp8 per-tensor")
    # row-wise Q/K
    rq8, eq = dta.fp8_quant_rows_pow2(q)
    rk8, ek = dta.fp8_quant_rows_pow2(k)
    o8, l8 = dta.attn_fwd_fp8_rows(rq8, rk8, v8, eq, ek, sv, scale)
    torch.cuda.synchronize()
    o_dq, l_dq = oracle.attention_fp8_rows(rq8.cpu().numpy(), rk8.cpu().numpy(), v8.cpu().numpy(),
                                           eq.cpu().numpy(), ek.cpu().numpy(), float(sv.item()),
                                           scale)
    _gates(o8, l8, o_bf, o_dq, l_dq, "random fp8 rows")
    o_st, bd = fp8_p_rounding_bound(deq_rows(rq8, eq), deq_rows(rk8, ek),
                                    deq_per_tensor(v8, float(sv.item())), scale,
                                    p_scale=KERNEL_P_SCALE)
    assert_within_bound(o8, o_st, bd, "random fp8 rows")
    # row-wise Q/K/V with per-block P scales
    rv8, ev = dta.fp8_quant_rows_pow2(v)
    o8, l8 = dta.attn_fwd_fp8_rows_v(rq8, rk8, rv8, eq, ek, ev, scale)
    torch.cuda.synchronize()
    o_dq, l_dq = oracle.attention_fp8_rows_v(rq8.cpu().numpy(), rk8.cpu().numpy(),
                                             rv8.cpu().numpy(), eq.cpu().numpy(),
                                             ek.cpu().numpy(), ev.cpu().numpy(), scale,
                                             block=KERNEL_P_BLOCK)
    _gates(o8, l8, o_bf, o_dq, l_dq, "random fp8 rows_v")
    ev_i = ev.cpu().numpy().astype(np.int64).reshape(B, H, Nkv) - 127
    o_st, bd = fp8_p_rounding_bound(deq_rows(rq8, eq), deq_rows(rk8, ek), deq_rows(rv8, ev), scale,
                                    vq=oracle.e4m3_decode(rv8.cpu().numpy()), ev=ev_i,
                                    block=KERNEL_P_BLOCK)
    assert_within_bound(o8, o_st, bd, "random fp8 rows_v")
