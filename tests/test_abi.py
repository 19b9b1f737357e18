"""The C ABI: libdta.so loads, exports every symbol include/dta.h declares,
and rejects bad arguments before any HIP call (runs without a GPU)."""

import ctypes
import os
import re

import pytest

from diffusion_transformer_attention_flash_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dta.h")

P = ctypes.c_void_p
GOOD = ctypes.c_void_p(0x10000)          # 16-byte aligned, never dereferenced
ODD = ctypes.c_void_p(0x10008)           # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_header_matches_binding_table():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_workspace_size():
    lib = _lib.lib()
    for s in (0, -1, -2, -3, -4, 99):
        assert lib.dta_status_str(s)
    assert lib.dta_ws_bytes() >= 16 * 1024


def test_attn_fwd_validation():
    f = _lib.lib().attn_fwd
    ok = (GOOD, GOOD, GOOD, GOOD, GOOD)
    assert f(None, GOOD, GOOD, GOOD, GOOD, 1, 1, 1, 1, 128, 0.1, None) == _lib.DTA_EINVAL
    assert f(*ok, 0, 1, 1, 1, 128, 0.1, None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 0, 128, 0.1, None) == _lib.DTA_EINVAL       # empty K/V
    assert f(*ok, 1, 1, 0, 1, 128, 0.1, None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 1, 96, 0.1, None) == _lib.DTA_EUNSUPPORTED
    assert f(*ok, 1, 1, 1, 1, 128, -0.5, None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 1, 128, float("nan"), None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 1, 128, float("inf"), None) == _lib.DTA_EINVAL
    assert f(ODD, GOOD, GOOD, GOOD, GOOD, 1, 1, 1, 1, 128, 0.1, None) == _lib.DTA_EALIGN
    assert f(GOOD, GOOD, GOOD, GOOD, ctypes.c_void_p(0x10002), 1, 1, 1, 1, 64, 0.1, None) == _lib.DTA_EALIGN


def test_attn_fwd_fp8_validation():
    f = _lib.lib().attn_fwd_fp8
    assert f(GOOD, GOOD, GOOD, None, GOOD, GOOD, 1, 1, 1, 1, 128, 0.1, None) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 1, 1, 1, 1, 80, 0.1, None) == _lib.DTA_EUNSUPPORTED
    assert f(GOOD, ODD, GOOD, GOOD, GOOD, GOOD, 1, 1, 1, 1, 64, 0.1, None) == _lib.DTA_EALIGN


def test_attn_merge_validation():
    f = _lib.lib().attn_merge
    assert f(GOOD, GOOD, 0, GOOD, GOOD, 1, 1, 1, 128, None) == _lib.DTA_EINVAL
    assert f(GOOD, None, 2, GOOD, GOOD, 1, 1, 1, 128, None) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, 2, GOOD, GOOD, 1, 1, 1, 32, None) == _lib.DTA_EUNSUPPORTED
    assert f(ODD, GOOD, 2, GOOD, GOOD, 1, 1, 1, 128, None) == _lib.DTA_EALIGN


def test_attn_fwd_accum_validation():
    f = _lib.lib().attn_fwd_accum
    ok = (GOOD, GOOD, GOOD, GOOD, GOOD)
    assert f(GOOD, GOOD, GOOD, GOOD, None, 1, 1, 1, 1, 128, 0.1, None) == _lib.DTA_EINVAL  # lse required
    assert f(None, GOOD, GOOD, GOOD, GOOD, 1, 1, 1, 1, 128, 0.1, None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 0, 128, 0.1, None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 1, 128, -1.0, None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 1, 96, 0.1, None) == _lib.DTA_EUNSUPPORTED
    assert f(GOOD, GOOD, GOOD, ODD, GOOD, 1, 1, 1, 1, 128, 0.1, None) == _lib.DTA_EALIGN
    assert f(GOOD, GOOD, GOOD, GOOD, ctypes.c_void_p(0x10002), 1, 1, 1, 1, 64, 0.1, None) == _lib.DTA_EALIGN


def test_attn_merge_into_validation():
    f = _lib.lib().attn_merge_into
    assert f(GOOD, None, GOOD, GOOD, 1, 1, 1, 128, None) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, GOOD, None, 1, 1, 1, 128, None) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, GOOD, GOOD, 1, 0, 1, 128, None) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, GOOD, GOOD, 1, 1, 1, 48, None) == _lib.DTA_EUNSUPPORTED
    assert f(GOOD, GOOD, ODD, GOOD, 1, 1, 1, 128, None) == _lib.DTA_EALIGN


def test_fbcache_step_validation():
    f = _lib.lib().fbcache_step
    ok = (GOOD, GOOD, 100, 0.08, GOOD, GOOD, 100, GOOD, GOOD, GOOD, None)
    assert f(None, *ok[1:]) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, 0, 0.08, GOOD, GOOD, 100, GOOD, GOOD, GOOD, None) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, 100, 0.08, GOOD, GOOD, 0, GOOD, GOOD, GOOD, None) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, 100, 0.08, GOOD, GOOD, 100, GOOD, None, GOOD, None) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, 100, 0.08, GOOD, GOOD, 100, GOOD, GOOD, None, None) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, 100, 0.08, ODD, GOOD, 100, GOOD, GOOD, GOOD, None) == _lib.DTA_EALIGN
    assert f(GOOD, GOOD, 100, 0.08, GOOD, GOOD, 100, GOOD, ctypes.c_void_p(0x10002), GOOD,
             None) == _lib.DTA_EALIGN


def test_fp8_rows_validation():
    lib = _lib.lib()
    assert lib.fp8_quant_rows_pow2(GOOD, 0, 128, GOOD, GOOD, None) == _lib.DTA_EINVAL
    assert lib.fp8_quant_rows_pow2(GOOD, 4, 12, GOOD, GOOD, None) == _lib.DTA_EINVAL   # row_len % 8
    assert lib.fp8_quant_rows_pow2(GOOD, 4, 128, GOOD, None, None) == _lib.DTA_EINVAL
    assert lib.fp8_quant_rows_pow2(ODD, 4, 128, GOOD, GOOD, None) == _lib.DTA_EALIGN
    f = lib.attn_fwd_fp8_rows
    ok = (GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD)
    assert f(GOOD, GOOD, GOOD, None, GOOD, GOOD, GOOD, GOOD, 1, 1, 1, 1, 128, 0.1, None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 0, 128, 0.1, None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 1, 96, 0.1, None) == _lib.DTA_EUNSUPPORTED
    assert f(ODD, *ok[1:], 1, 1, 1, 1, 128, 0.1, None) == _lib.DTA_EALIGN


def test_fp8_rows_v_validation():
    lib = _lib.lib()
    f = lib.attn_fwd_fp8_rows_v
    ok = (GOOD,) * 8                                   # q8 k8 v8 q_e k_e v_e o lse
    for i in range(7):                                 # every required pointer
        args = list(ok)
        args[i] = None
        assert f(*args, 1, 1, 1, 1, 128, 0.1, None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 0, 128, 0.1, None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 1, 128, -1.0, None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 1, 128, float("nan"), None) == _lib.DTA_EINVAL
    assert f(*ok, 1, 1, 1, 1, 96, 0.1, None) == _lib.DTA_EUNSUPPORTED
    assert f(ODD, *ok[1:], 1, 1, 1, 1, 128, 0.1, None) == _lib.DTA_EALIGN
    assert f(*ok[:6], ODD, ok[7], 1, 1, 1, 1, 128, 0.1, None) == _lib.DTA_EALIGN


def test_layout_validation():
    lib = _lib.lib()
    I = ctypes.c_int
    two = (I * 2)(3, 4)
    pads = (I * 2)(3, 5)
    bad_pads = (I * 2)(2, 5)                      # padded < lens
    zeros = (I * 2)(0, 0)
    assert lib.seq_concat(GOOD, GOOD, 0, two, pads, 1, 2, 128, None) == _lib.DTA_EINVAL
    assert lib.seq_concat(GOOD, GOOD, 65, two, pads, 1, 2, 128, None) == _lib.DTA_EINVAL
    assert lib.seq_concat(GOOD, GOOD, 2, None, pads, 1, 2, 128, None) == _lib.DTA_EINVAL
    assert lib.seq_concat(GOOD, GOOD, 2, two, bad_pads, 1, 2, 128, None) == _lib.DTA_EINVAL
    assert lib.seq_concat(GOOD, GOOD, 2, zeros, pads, 1, 2, 128, None) == _lib.DTA_EINVAL
    assert lib.seq_split(GOOD, GOOD, 2, two, None, 1, 2, 100, None) == _lib.DTA_EINVAL  # D % 8
    assert lib.seq_split(GOOD, ODD, 2, two, None, 1, 2, 128, None) == _lib.DTA_EALIGN
    assert lib.head_concat(GOOD, GOOD, 2, zeros, 1, 8, 128, None) == _lib.DTA_EINVAL  # heads >= 1
    one_empty = (I * 2)(3, 0)                     # a single part with no heads
    assert lib.head_concat(GOOD, GOOD, 2, one_empty, 1, 8, 128, None) == _lib.DTA_EINVAL
    assert lib.head_split(GOOD, GOOD, 2, one_empty, 1, 8, 128, None) == _lib.DTA_EINVAL
    assert lib.seq_concat(GOOD, GOOD, 2, (I * 2)(3, 0), None, 1, 2, 128, None) == _lib.DTA_EINVAL
    assert lib.head_split(None, GOOD, 2, two, 1, 8, 128, None) == _lib.DTA_EINVAL
    assert lib.head_split(ODD, GOOD, 2, two, 1, 8, 128, None) == _lib.DTA_EALIGN


def test_reductions_validation():
    lib = _lib.lib()
    f = lib.residual_diff_noalloc
    assert f(None, GOOD, 10, GOOD, None) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, 10, None, None) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, 0, GOOD, None) == _lib.DTA_EINVAL
    assert f(GOOD, GOOD, 1 << 62, GOOD, None) == _lib.DTA_EINVAL      # beyond the limit
    assert f(ODD, GOOD, 10, GOOD, None) == _lib.DTA_EALIGN
    assert f(GOOD, GOOD, 10, ctypes.c_void_p(0x10002), None) == _lib.DTA_EALIGN
    assert lib.residual_diff(GOOD, GOOD, 0, GOOD, GOOD, None) == _lib.DTA_EINVAL
    assert lib.residual_diff(GOOD, GOOD, 10, GOOD, None, None) == _lib.DTA_EINVAL
    assert lib.residual_diff(ODD, GOOD, 10, GOOD, GOOD, None) == _lib.DTA_EALIGN
    assert lib.fp8_quant_per_tensor(GOOD, 0, GOOD, GOOD, GOOD, None) == _lib.DTA_EINVAL
    assert lib.fp8_quant_per_tensor(GOOD, 10, ODD, GOOD, GOOD, None) == _lib.DTA_EALIGN


def test_quant_multi_validation():
    lib = _lib.lib()
    P = ctypes.c_void_p
    xs = (P * 3)(0x10000, 0x20000, 0x30000)
    x8s = (P * 3)(0x40000, 0x50000, 0x60000)
    ns = (ctypes.c_int64 * 3)(10, 20, 30)
    cast = lambda a: ctypes.cast(a, P)
    call = lambda cnt, x=xs, n=ns, x8=x8s, ds=GOOD, ws=GOOD: lib.fp8_quant_per_tensor_multi(
        cnt, cast(x) if x is not None else None, cast(n) if n is not None else None,
        cast(x8) if x8 is not None else None, ds, ws, None)
    assert call(0) == _lib.DTA_EINVAL                       # count out of range
    assert call(5) == _lib.DTA_EINVAL
    assert call(3, x=None) == _lib.DTA_EINVAL
    assert call(3, n=None) == _lib.DTA_EINVAL
    assert call(3, ds=None) == _lib.DTA_EINVAL
    assert call(3, ws=None) == _lib.DTA_EINVAL
    assert call(3, n=(ctypes.c_int64 * 3)(10, 0, 30)) == _lib.DTA_EINVAL   # a size < 1
    assert call(3, x=(P * 3)(0x10000, None, 0x30000)) == _lib.DTA_EINVAL   # a null tensor
    assert call(3, x8=(P * 3)(0x40000, 0x50008, 0x60000)) == _lib.DTA_EALIGN
    assert call(3, ds=ctypes.c_void_p(0x10002)) == _lib.DTA_EALIGN
    assert call(3, ws=ODD) == _lib.DTA_EALIGN


def test_binding_rejects_cpu_tensors():
    import torch
    import diffusion_transformer_attention_flash_amd as dta
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dta.attn_fwd(q, q, q)
    with pytest.raises(ValueError):
        dta.residual_diff(q, q)


def test_missing_library_raises(monkeypatch):
    """No fallback: with the shared library absent the binding raises."""
    monkeypatch.setattr(_lib, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libdta.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_host_tensors_are_rejected():
    """The binding takes device tensors only; host tensors raise before any
    library call (there is no CPU path)."""
    import torch
    import diffusion_transformer_attention_flash_amd as dta
    q = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        dta.attn_fwd(q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        dta.residual_diff(q, q)
    with pytest.raises(ValueError, match="GPU"):
        dta.fp8_quant_per_tensor(q)


def test_binding_checks_every_output_before_the_device():
    """A caller-supplied output of the wrong shape or dtype raises, naming
    it, before any device check or library call (so this runs on host
    tensors: shapes and dtypes are checked first)."""
    import torch
    import diffusion_transformer_attention_flash_amd as dta
    bf, f32, u8, i32 = torch.bfloat16, torch.float32, torch.uint8, torch.int32
    q = torch.zeros(1, 2, 8, 64, dtype=bf)
    q8 = torch.zeros(1, 2, 8, 64, dtype=u8)
    e8 = torch.zeros(1, 2, 8, dtype=u8)
    ds3 = torch.zeros(3, dtype=f32)
    ds1 = torch.zeros(1, dtype=f32)
    good_o, good_l = torch.zeros(1, 2, 8, 64, dtype=bf), torch.zeros(1, 2, 8, dtype=f32)
    short_o, short_l = torch.zeros(1, 2, 7, 64, dtype=bf), torch.zeros(1, 2, 7, dtype=f32)
    cases = [
        (lambda: dta.attn_fwd(q, q, q, o=short_o), ValueError, "o"),
        (lambda: dta.attn_fwd(q, q, q, o=good_o.float()), TypeError, "o"),
        (lambda: dta.attn_fwd(q, q, q, lse=short_l), ValueError, "lse"),
        (lambda: dta.attn_merge(q[None].expand(2, -1, -1, -1, -1).contiguous(),
                                good_l[None].expand(2, -1, -1, -1).contiguous(), o=short_o),
         ValueError, "o"),
        (lambda: dta.attn_merge(q[None].contiguous(), good_l[None].contiguous(), lse=short_l),
         ValueError, "lse"),
        (lambda: dta.attn_fwd_accum(q, q, q, short_o, good_l), ValueError, "o"),
        (lambda: dta.attn_fwd_accum(q, q, q, good_o, good_l.double()), TypeError, "lse"),
        (lambda: dta.attn_merge_into(good_o, short_l, good_o, good_l), ValueError, "lse"),
        (lambda: dta.attn_merge_into(good_o, good_l, short_o, good_l), ValueError, "o_part"),
        (lambda: dta.residual_diff(q, q, out=torch.zeros(2, dtype=f32)), ValueError, "out"),
        (lambda: dta.residual_diff(q, q, out=torch.zeros((), dtype=bf)), TypeError, "out"),
        (lambda: dta.fbcache_step(q, q, 0.1, q.clone(), q, diff=torch.zeros(2, dtype=f32)),
         ValueError, "diff"),
        (lambda: dta.fbcache_step(q, q, 0.1, q.clone(), q, use_cache=torch.zeros((), dtype=f32)),
         TypeError, "use_cache"),
        (lambda: dta.fp8_quant_per_tensor(q, x8=torch.zeros(10, dtype=u8)), ValueError, "x8"),
        (lambda: dta.fp8_quant_per_tensor(q, descale=torch.zeros(2, dtype=f32)), ValueError,
         "descale"),
        (lambda: dta.fp8_quant_per_tensor_multi([q, q], descale=torch.zeros(1, dtype=f32)),
         ValueError, "descale"),
        (lambda: dta.fp8_quant_per_tensor_multi([q], x8s=[torch.zeros(5, dtype=u8)]),
         ValueError, "x8s[0]"),
        (lambda: dta.attn_fwd_fp8(q8, q8, q8, ds1), ValueError, "descale"),
        (lambda: dta.attn_fwd_fp8(q8, q8, q8, ds3, o=short_o), ValueError, "o"),
        (lambda: dta.attn_fwd_fp8(q8, q8, q8, ds3, lse=good_l.to(bf)), TypeError, "lse"),
        (lambda: dta.fp8_quant_rows_pow2(q, e8m0=torch.zeros(3, dtype=u8)), ValueError, "e8m0"),
        (lambda: dta.fp8_quant_rows_pow2(q, x8=torch.zeros(3, dtype=u8)), ValueError, "x8"),
        (lambda: dta.attn_fwd_fp8_rows(q8, q8, q8, e8, e8, ds3), ValueError, "v_descale"),
        (lambda: dta.attn_fwd_fp8_rows(q8, q8, q8, e8[:, :1], e8, ds1), ValueError, "q_e8m0"),
        (lambda: dta.attn_fwd_fp8_rows(q8, q8, q8, e8, e8, ds1, o=short_o), ValueError, "o"),
        (lambda: dta.attn_fwd_fp8_rows_v(q8, q8, q8, e8, e8, e8[:, :1]), ValueError, "v_e8m0"),
        (lambda: dta.attn_fwd_fp8_rows_v(q8, q8, q8, e8, e8, e8, lse=short_l), ValueError, "lse"),
        (lambda: dta.seq_concat(q.view(-1), [4, 4], 1, 2, 64, out=torch.zeros(3, dtype=bf)),
         ValueError, "out"),
        (lambda: dta.head_split(q, [1, 1], parts=torch.zeros(3, dtype=bf)), ValueError, "parts"),
    ]
    for fn, exc, name in cases:
        with pytest.raises(exc, match=re.escape(name)):
            fn()
