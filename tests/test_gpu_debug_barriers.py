"""The attention kernels built with a workgroup barrier at every point where
they hand LDS from one phase to the next (libdta_debug.so, DTA_DEBUG_BARRIERS)
against the normal build: the barriers change no arithmetic, so every output
must be bit-identical. A race on reused LDS (the staged O epilogues, the fp8
kernel's three rotating K/V buffers under skewed waves) would show up as a
difference."""

import ctypes
import os

import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
from diffusion_transformer_attention_flash_amd import _lib, build
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _debug_lib():
    if not os.path.exists(build.DEBUG_LIB_PATH):
        pytest.fail("libdta_debug.so is not built (run __graft_entry__.build())")
    h = ctypes.CDLL(build.DEBUG_LIB_PATH)
    for name, (res, args) in _lib.SIGNATURES.items():
        f = getattr(h, name)
        f.restype, f.argtypes = res, args
    return h


P = ctypes.c_void_p
p = lambda t: P(t.data_ptr())  # noqa: E731


def _stream():
    return P(torch.cuda.current_stream().cuda_stream)


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("B,H,Nq,Nkv", [(1, 2, 300, 1), (1, 2, 300, 65), (1, 2, 513, 130),
                                        (1, 2, 300, 192), (2, 1, 257, 385), (1, 24, 4608, 4608)])
def test_bf16_and_ring_match_the_extra_barrier_build(B, H, Nq, Nkv):
    print("CASE debug barriers bf16", B, H, Nq, Nkv, flush=True)
    dbg = _debug_lib()
    q, k, v = workloads.make_qkv(41, B, H, Nq, Nkv, 128, device=DEV)
    o, lse = dta.attn_fwd(q, k, v, 128 ** -0.5)
    o2, l2 = torch.empty_like(o), torch.empty_like(lse)
    assert dbg.attn_fwd(p(q), p(k), p(v), p(o2), p(l2), B, H, Nq, Nkv, 128, 128 ** -0.5,
                        _stream()) == 0
    # a two-chunk fused ring (the ACCUM epilogue)
    cut = max(1, Nkv // 3)
    (k1, v1), (k2, v2) = workloads.split_kv(k, v, [cut, Nkv - cut]) if Nkv > 1 else \
        ((k, v), (k, v))
    orr, lr = dta.attn_fwd(q, k1, v1, 128 ** -0.5)
    dta.attn_fwd_accum(q, k2, v2, orr, lr, 128 ** -0.5)
    orr2, lr2 = dta.attn_fwd(q, k1, v1, 128 ** -0.5)
    assert dbg.attn_fwd_accum(p(q), p(k2), p(v2), p(orr2), p(lr2), B, H, Nq, k2.shape[2], 128,
                              128 ** -0.5, _stream()) == 0
    torch.cuda.synchronize()
    assert _same(o, o2) and _same(lse, l2)
    assert _same(orr, orr2) and _same(lr, lr2)


@pytest.mark.parametrize("Nkv", [1, 64, 65, 128, 150, 192, 256, 320, 385, 4608])
def test_fp8_variants_match_the_extra_barrier_build(Nkv):
    print("CASE debug barriers fp8", Nkv, flush=True)
    dbg = _debug_lib()
    B, H, Nq, D = 1, 2, 513, 128
    q, k, v = workloads.make_qkv(43, B, H, Nq, Nkv, D, device=DEV)
    (q8, k8, v8), ds = dta.fp8_quant_per_tensor_multi([q, k, v])
    rq8, eq = dta.fp8_quant_rows_pow2(q)
    rk8, ek = dta.fp8_quant_rows_pow2(k)
    rv8, ev = dta.fp8_quant_rows_pow2(v)
    scale = D ** -0.5
    outs = [dta.attn_fwd_fp8(q8, k8, v8, ds, scale),
            dta.attn_fwd_fp8_rows(rq8, rk8, v8, eq, ek, ds[2:3], scale),
            dta.attn_fwd_fp8_rows_v(rq8, rk8, rv8, eq, ek, ev, scale)]
    dbg_outs = []
    for i in range(3):
        o2 = torch.empty((B, H, Nq, D), dtype=torch.bfloat16, device=DEV)
        l2 = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
        if i == 0:
            st = dbg.attn_fwd_fp8(p(q8), p(k8), p(v8), p(ds), p(o2), p(l2), B, H, Nq, Nkv, D,
                                  scale, _stream())
        elif i == 1:
            st = dbg.attn_fwd_fp8_rows(p(rq8), p(rk8), p(v8), p(eq), p(ek), P(ds.data_ptr() + 8),
                                       p(o2), p(l2), B, H, Nq, Nkv, D, scale, _stream())
        else:
            st = dbg.attn_fwd_fp8_rows_v(p(rq8), p(rk8), p(rv8), p(eq), p(ek), p(ev), p(o2), p(l2),
                                         B, H, Nq, Nkv, D, scale, _stream())
        assert st == 0
        dbg_outs.append((o2, l2))
    torch.cuda.synchronize()
    for (o, l), (o2, l2) in zip(outs, dbg_outs):
        assert _same(o, o2) and _same(l, l2)
