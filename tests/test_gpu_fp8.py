"""GPU parity of the fp8 dynamic-quantisation attention variant."""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
import oracle
import workloads
from helpers import (FP8_O_MEAN_ABS, FP8_REL_L2_VS_BF16, FP8_REL_L2_VS_BF16_PEAKED,
                     FP8_REL_L2_VS_DEQUANT, KERNEL_P_SCALE, LSE_ABS, assert_within_bound,
                     deq_per_tensor, fp8_p_rounding_bound, head_groups, rel_l2, take_rows, to64)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _quant3(q, k, v):
    q8, sq = dta.fp8_quant_per_tensor(q)
    k8, sk = dta.fp8_quant_per_tensor(k)
    v8, sv = dta.fp8_quant_per_tensor(v)
    ds = torch.cat([sq, sk, sv])
    return q8, k8, v8, ds


def _check(o8, l8, q, k, v, q8, k8, v8, ds, scale, rows=None, what="",
           gate_bf16=FP8_REL_L2_VS_BF16):
    """Gates against the bf16-input oracle and the dequantised oracle, and
    the elementwise P-rounding bound against exact attention on the
    dequantised inputs. rows None: every row; else [H, r] rows per head."""
    dsc = ds.cpu().tolist()
    q8n, k8n, v8n = (t.cpu().numpy() for t in (q8, k8, v8))
    acc = {key: [] for key in ("o", "l", "bf", "dq", "ldq", "star", "bound")}
    for hs, r in head_groups(rows, q.shape[1]):
        o_dq, l_dq = oracle.attention_fp8(q8n[:, hs], k8n[:, hs], v8n[:, hs], dsc, scale, rows=r)
        o_bf, _ = oracle.attention(q[:, hs].cpu(), k[:, hs].cpu(), v[:, hs].cpu(), scale, rows=r)
        o_st, bd = fp8_p_rounding_bound(deq_per_tensor(q8n[:, hs], dsc[0]),
                                        deq_per_tensor(k8n[:, hs], dsc[1]),
                                        deq_per_tensor(v8n[:, hs], dsc[2]), scale,
                                        p_scale=KERNEL_P_SCALE, rows=r)
        for key, val in (("o", to64(take_rows(o8, hs, r))), ("l", to64(take_rows(l8, hs, r))),
                         ("bf", o_bf), ("dq", o_dq), ("ldq", l_dq), ("star", o_st),
                         ("bound", bd)):
            acc[key].append(val)
    a = {key: np.concatenate(val, axis=1) for key, val in acc.items()}
    o8, l8 = a["o"], a["l"]
    assert np.isfinite(o8).all() and np.isfinite(l8).all()
    mean_abs = np.abs(o8 - a["bf"]).mean()
    r_bf = rel_l2(o8, a["bf"])
    r_dq = rel_l2(o8, a["dq"])
    e_l = np.abs(l8 - a["ldq"]).max()
    msg = "%s: O mean-abs %.3e vs bf16 oracle, rel-L2 %.3e (bf16) %.3e (dequant), LSE %.3e" % (
        what, mean_abs, r_bf, r_dq, e_l)
    print(msg)
    assert mean_abs <= FP8_O_MEAN_ABS, msg
    assert r_bf <= gate_bf16, msg
    assert r_dq <= FP8_REL_L2_VS_DEQUANT, msg
    assert e_l <= LSE_ABS, msg
    assert_within_bound(o8, a["star"], a["bound"], what)


@pytest.mark.parametrize("B,H,Nq,Nkv,D", [(1, 2, 300, 300, 128), (1, 3, 200, 131, 64),
                                          (1, 1, 64, 1, 128), (2, 1, 97, 640, 128)])
def test_fp8_attention_shapes(B, H, Nq, Nkv, D):
    print("CASE fp8 shape", B, H, Nq, Nkv, D, flush=True)
    q, k, v = workloads.make_qkv(21, B, H, Nq, Nkv, D, device=DEV)
    q8, k8, v8, ds = _quant3(q, k, v)
    o8, l8 = dta.attn_fwd_fp8(q8, k8, v8, ds, D ** -0.5)
    torch.cuda.synchronize()
    _check(o8, l8, q, k, v, q8, k8, v8, ds, D ** -0.5, what="fp8 shape")


def test_fp8_attention_peaked():
    print("CASE fp8 peaked", flush=True)
    q, k, v = workloads.make_qkv(23, 1, 2, 256, 512, 128, device=DEV, q_gain=4.0)
    q8, k8, v8, ds = _quant3(q, k, v)
    o8, l8 = dta.attn_fwd_fp8(q8, k8, v8, ds, 128 ** -0.5)
    torch.cuda.synchronize()
    _check(o8, l8, q, k, v, q8, k8, v8, ds, 128 ** -0.5, what="fp8 peaked",
           gate_bf16=FP8_REL_L2_VS_BF16_PEAKED)


def test_fp8_flux_1024_all_rows():
    c = workloads.CONFIGS["flux_1024_fp8"]
    print("CASE fp8 flux_1024 (all rows)", flush=True)
    q, k, v = workloads.workload_qkv("flux_1024_fp8", device=DEV)
    q8, k8, v8, ds = _quant3(q, k, v)
    o8, l8 = dta.attn_fwd_fp8(q8, k8, v8, ds, c["D"] ** -0.5)
    torch.cuda.synchronize()
    _check(o8, l8, q, k, v, q8, k8, v8, ds, c["D"] ** -0.5, what="fp8 flux (all rows)")


def test_fp8_video_length_rows_per_head():
    """The HunyuanVideo 720p x 129-frame sequence length (119 056 tokens: 1861
    K/V tiles, the last one 16 keys) on two heads of its recipe, 256 query
    rows per head (forced edge rows, one row in each 32-row block dealt to
    the head): the longest K/V loop of the workloads, with its running max,
    rare rescales and float32 row sums. Two heads keep the oracle's
    quantisation of the whole tensors within seconds."""
    c = workloads.CONFIGS["hunyuan_720p_129f"]
    N, D = c["N"], c["D"]
    print("CASE fp8 video length, 2 heads", flush=True)
    q, k, v = workloads.make_qkv(c["config"], 1, 2, N, N, D, device=DEV)
    q8, k8, v8, ds = _quant3(q, k, v)
    o8, l8 = dta.attn_fwd_fp8(q8, k8, v8, ds, D ** -0.5)
    torch.cuda.synchronize()
    rows = workloads.sample_rows_per_head(c["config"], N, 2, 256, c["n_text"])
    _check(o8, l8, q, k, v, q8, k8, v8, ds, D ** -0.5, rows=rows, what="fp8 video length")


@pytest.mark.parametrize("Nkv", [1, 40, 64, 65, 128, 150, 192, 256, 300, 320, 385])
def test_fp8_attention_tile_counts(Nkv):
    """K/V lengths of 1 to 7 tiles of 64 keys, full and ragged last tile: the
    8-wave D = 128 kernel rotates three LDS buffers and its skewed waves finish
    the last tile's P.V after the loop, so every residue of the tile count
    mod 3 and both tail kinds are covered."""
    print("CASE fp8 tile count", Nkv, flush=True)
    q, k, v = workloads.make_qkv(29, 1, 2, 300, Nkv, 128, device=DEV)
    q8, k8, v8, ds = _quant3(q, k, v)
    o8, l8 = dta.attn_fwd_fp8(q8, k8, v8, ds, 128 ** -0.5)
    torch.cuda.synchronize()
    _check(o8, l8, q, k, v, q8, k8, v8, ds, 128 ** -0.5, what="fp8 Nkv=%d" % Nkv)


@pytest.mark.parametrize("Nkv", [300, 1024])
def test_fp8_query_position_invariance(Nkv):
    """A query's O and LSE do not depend on which wave computes it. Rolling
    the queries by 128 rows moves every query between the first and the
    second half of a 256-query workgroup (the on-time and the skewed waves);
    O and LSE must roll bit for bit."""
    print("CASE fp8 query roll", Nkv, flush=True)
    q, k, v = workloads.make_qkv(31, 1, 2, 512, Nkv, 128, device=DEV)
    q8, k8, v8, ds = _quant3(q, k, v)
    o_a, l_a = dta.attn_fwd_fp8(q8, k8, v8, ds, 128 ** -0.5)
    o_b, l_b = dta.attn_fwd_fp8(torch.roll(q8, 128, dims=2).contiguous(), k8, v8, ds,
                                128 ** -0.5)
    torch.cuda.synchronize()
    assert torch.equal(torch.roll(o_a, 128, dims=2), o_b)
    assert torch.equal(torch.roll(l_a, 128, dims=2), l_b)
