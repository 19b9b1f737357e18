"""The ABI's optional LSE output (include/dta.h: attn_fwd, attn_fwd_fp8 and
attn_merge accept lse == NULL and then do not write it), through the C ABI:
O must be bit-identical to the call that writes LSE, at a ragged shape, for
both attention epilogues (D = 128: 8 waves, staged O; D = 64: 4 waves)."""

import ctypes

import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
from diffusion_transformer_attention_flash_amd import _lib
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"
P = ctypes.c_void_p


def _p(t):
    return P(t.data_ptr())


def _stream():
    return P(torch.cuda.current_stream().cuda_stream)


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("D", [64, 128])
def test_attn_fwd_without_lse(D):
    B, H, Nq, Nkv = 1, 3, 517, 300
    print("CASE attn_fwd lse=NULL", B, H, Nq, Nkv, D, flush=True)
    q, k, v = workloads.make_qkv(61, B, H, Nq, Nkv, D, device=DEV)
    o_ref, _ = dta.attn_fwd(q, k, v, D ** -0.5)
    o = torch.full_like(o_ref, float("nan"))
    assert _lib.lib().attn_fwd(_p(q), _p(k), _p(v), _p(o), None, B, H, Nq, Nkv, D, D ** -0.5,
                               _stream()) == 0
    torch.cuda.synchronize()
    assert _same(o, o_ref)


def test_attn_fwd_fp8_without_lse():
    B, H, Nq, Nkv, D = 1, 2, 517, 300, 128
    print("CASE attn_fwd_fp8 lse=NULL", B, H, Nq, Nkv, D, flush=True)
    q, k, v = workloads.make_qkv(62, B, H, Nq, Nkv, D, device=DEV)
    (q8, k8, v8), ds = dta.fp8_quant_per_tensor_multi([q, k, v])
    o_ref, _ = dta.attn_fwd_fp8(q8, k8, v8, ds, D ** -0.5)
    o = torch.full_like(o_ref, float("nan"))
    assert _lib.lib().attn_fwd_fp8(_p(q8), _p(k8), _p(v8), _p(ds), _p(o), None, B, H, Nq, Nkv,
                                   D, D ** -0.5, _stream()) == 0
    torch.cuda.synchronize()
    assert _same(o, o_ref)


def test_attn_merge_without_lse():
    n, B, H, Nq, D = 3, 1, 2, 333, 128
    print("CASE attn_merge lse=NULL", n, B, H, Nq, D, flush=True)
    g = torch.Generator().manual_seed(63)
    o_parts = torch.randn((n, B, H, Nq, D), generator=g).to(torch.bfloat16).to(DEV)
    l_parts = (torch.randn((n, B, H, Nq), generator=g) * 4).to(DEV)
    o_ref, _ = dta.attn_merge(o_parts, l_parts)
    o = torch.full_like(o_ref, float("nan"))
    assert _lib.lib().attn_merge(_p(o_parts), _p(l_parts), n, _p(o), None, B, H, Nq, D,
                                 _stream()) == 0
    torch.cuda.synchronize()
    assert _same(o, o_ref)
