"""Every K/V tail: Nkv = 1 .. 129 (each residue of the 64-key tile, one and
two full tiles, and one key past them) through the bf16 kernel (D = 64 and
128), the per-tensor and the row-wise Q/K/V fp8 kernels, and a two-chunk
fused ring cut after every key of a 130-key sequence; each case against the
oracle. The query side is one ragged tile (37 rows) of two heads."""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
import oracle
import workloads
from helpers import (KERNEL_P_BLOCK, KERNEL_P_SCALE, assert_bf16_attention, assert_within_bound,
                     deq_per_tensor, deq_rows, fp8_p_rounding_bound)

pytestmark = pytest.mark.gpu
DEV = "cuda"
B, H, NQ = 1, 2, 37
NKV = range(1, 130)


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_every_kv_length(D):
    scale = D ** -0.5
    for nkv in NKV:
        print("CASE bf16 tail", D, nkv, flush=True)
        q, k, v = workloads.make_qkv(4000 + nkv, B, H, NQ, nkv, D, device=DEV, q_gain=2.0)
        o, lse = dta.attn_fwd(q, k, v, scale)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
        assert_bf16_attention(o, lse, o_ref, lse_ref, "bf16 D=%d Nkv=%d" % (D, nkv))


def test_fp8_every_kv_length():
    D = 128
    scale = D ** -0.5
    for nkv in NKV:
        print("CASE fp8 tail", nkv, flush=True)
        q, k, v = workloads.make_qkv(5000 + nkv, B, H, NQ, nkv, D, device=DEV)
        (q8, k8, v8), ds = dta.fp8_quant_per_tensor_multi([q, k, v])
        o8, l8 = dta.attn_fwd_fp8(q8, k8, v8, ds, scale)
        rq8, eq = dta.fp8_quant_rows_pow2(q)
        rk8, ek = dta.fp8_quant_rows_pow2(k)
        rv8, ev = dta.fp8_quant_rows_pow2(v)
        ov, lv = dta.attn_fwd_fp8_rows_v(rq8, rk8, rv8, eq, ek, ev, scale)
        torch.cuda.synchronize()
        dsc = ds.cpu().tolist()
        o_st, bd = fp8_p_rounding_bound(deq_per_tensor(q8, dsc[0]), deq_per_tensor(k8, dsc[1]),
                                        deq_per_tensor(v8, dsc[2]), scale,
                                        p_scale=KERNEL_P_SCALE)
        assert_within_bound(o8, o_st, bd, "fp8 per-tensor Nkv=%d" % nkv)
        _, l_dq = oracle.attention_fp8(q8.cpu().numpy(), k8.cpu().numpy(), v8.cpu().numpy(),
                                       dsc, scale)
        assert np.abs(l8.cpu().double().numpy() - l_dq).max() < 1e-3
        ev_i = ev.cpu().numpy().astype(np.int64).reshape(B, H, nkv) - 127
        o_st, bd = fp8_p_rounding_bound(deq_rows(rq8, eq), deq_rows(rk8, ek), deq_rows(rv8, ev),
                                        scale, vq=oracle.e4m3_decode(rv8.cpu().numpy()),
                                        ev=ev_i, block=KERNEL_P_BLOCK)
        assert_within_bound(ov, o_st, bd, "fp8 rows_v Nkv=%d" % nkv)


def test_fused_ring_every_cut():
    D, n = 128, 130
    scale = D ** -0.5
    q, k, v = workloads.make_qkv(6000, B, H, NQ, n, D, device=DEV, q_gain=2.0)
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    for cut in range(1, n):
        print("CASE ring cut", cut, flush=True)
        (k1, v1), (k2, v2) = workloads.split_kv(k, v, [cut, n - cut])
        o, lse = dta.attn_fwd(q, k1, v1, scale)
        dta.attn_fwd_accum(q, k2, v2, o, lse, scale)
        torch.cuda.synchronize()
        assert_bf16_attention(o, lse, o_ref, lse_ref, "ring cut %d" % cut)
