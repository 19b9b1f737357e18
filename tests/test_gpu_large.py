"""Tensors of more than 2^31 elements: every offset in the kernels is 64-bit.

The inputs are built so that the exact result has a closed form (no oracle
pass over billions of elements): mostly zeros or ones, with a few planted
values at offsets past 2^31 elements, where a 32-bit index would wrap.
Each test needs 7-18 GB of device memory and runs in about a second.
"""

import math

import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta

pytestmark = pytest.mark.gpu
DEV = "cuda"
TWO31 = 1 << 31


def _case(name, **kw):
    print("CASE", name, kw, flush=True)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_attention_keys_past_2_31_elements():
    """Two heads of 2^24 + 37 keys (D = 128): each head's K/V span more than
    2^31 elements, so head 1 starts past that offset and the last key of
    either head lies beyond it. All keys are zero except the last one, so a
    query q = (a, 0, ...) scores s* = scale*a on that key and 0 elsewhere:
        O = v_last e^s* / (e^s* + N - 1),  LSE = ln(e^s* + N - 1)."""
    H, N, D = 2, (1 << 24) + 37, 128
    assert N * D > TWO31
    _case("attn_fwd large", H=H, Nkv=N, D=D)
    scale = D ** -0.5
    k = torch.zeros((1, H, N, D), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    k[0, :, N - 1, 0] = 1.0
    c = [2.0, -3.0]
    for h in range(H):
        v[0, h, N - 1, :] = c[h]
    a = 188.0                                   # exact in bf16; s* = 16.6
    q = torch.zeros((1, H, 3, D), dtype=torch.bfloat16, device=DEV)
    q[0, :, 0, 0] = a                           # the last key dominates
    q[0, :, 2, 0] = -a                          # the last key nearly vanishes
    o, lse = dta.attn_fwd(q, k, v, scale)
    torch.cuda.synchronize()
    del k, v
    _free()
    for h in range(H):
        for r, s in ((0, scale * a), (1, 0.0), (2, -scale * a)):
            l_exact = math.exp(s) + (N - 1)
            o_exact = c[h] * math.exp(s) / l_exact
            got = o[0, h, r].float().cpu()
            assert torch.allclose(got, torch.full_like(got, o_exact), rtol=2 ** -7, atol=0), \
                (h, r, got[:4], o_exact)
            assert abs(float(lse[0, h, r]) - math.log(l_exact)) < 1e-4, (h, r, float(lse[0, h, r]))


def test_fp8_attention_keys_past_2_31_bytes():
    """The per-tensor fp8 kernel on the same construction as above, in E4M3
    codes (descales 1): K/V of two heads of 2^24 + 37 keys are 2.15e9 bytes
    each, all zero but the last key (k = 1, v = c_h); q = (192, 0, ...),
    0 or (-192, 0, ...). Only the last key carries a value, so O has no
    accumulation error: O = c_h w with w = e^s/(e^s + N - 1) up to the E4M3
    rounding of the kernel's 108 p (2^-4 relative, or 2^-10/(108 l) of |c_h|
    below E4M3's normal range, l the exact normaliser against the row max)
    and two bf16 roundings; LSE comes from the unrounded p."""
    H, N, D = 2, (1 << 24) + 37, 128
    assert N * D > TWO31
    _case("attn_fwd_fp8 large", H=H, Nkv=N, D=D)
    code = lambda x: int(torch.tensor([x]).to(torch.float8_e4m3fn).view(torch.uint8))  # noqa: E731
    scale = D ** -0.5
    k8 = torch.zeros((1, H, N, D), dtype=torch.uint8, device=DEV)
    v8 = torch.zeros_like(k8)
    k8[0, :, N - 1, 0] = code(1.0)
    c = [2.0, -3.0]
    for h in range(H):
        v8[0, h, N - 1, :] = code(c[h])
    q8 = torch.zeros((1, H, 3, D), dtype=torch.uint8, device=DEV)
    q8[0, :, 0, 0] = code(192.0)
    q8[0, :, 2, 0] = code(-192.0)
    ds = torch.ones(3, dtype=torch.float32, device=DEV)
    o, lse = dta.attn_fwd_fp8(q8, k8, v8, ds, scale)
    torch.cuda.synchronize()
    del k8, v8
    _free()
    for h in range(H):
        for r, s in ((0, scale * 192.0), (1, 0.0), (2, -scale * 192.0)):
            m = max(s, 0.0)
            l = math.exp(s - m) + (N - 1) * math.exp(-m)
            o_exact = c[h] * math.exp(s - m) / l
            bound = (2 ** -4 + 2 ** -8) * abs(o_exact) + 2 ** -10 * abs(c[h]) / (108.0 * l) + 1e-30
            got = o[0, h, r].double().cpu()
            assert float((got - o_exact).abs().max()) <= bound, (h, r, got[:4], o_exact, bound)
            assert abs(float(lse[0, h, r]) - (m + math.log(l))) < 1e-4, (h, r, float(lse[0, h, r]))


def test_merge_rows_past_2_31_elements():
    """Two partials of 2^23 + 5 rows x 128 (2.15e9 elements together): O_0 = 1,
    O_1 = 3, LSE_0 = 0, LSE_1 = ln 3, so O = (1 + 3*3) / 4 = 2.5 and
    LSE = ln 4 in every row."""
    rows, D = (1 << 23) + 5, 128
    assert 2 * rows * D > TWO31
    _case("attn_merge large", rows=rows, D=D)
    o_parts = torch.empty((2, 1, 1, rows, D), dtype=torch.bfloat16, device=DEV)
    o_parts[0].fill_(1.0)
    o_parts[1].fill_(3.0)
    l_parts = torch.empty((2, 1, 1, rows), dtype=torch.float32, device=DEV)
    l_parts[0].fill_(0.0)
    l_parts[1].fill_(math.log(3.0))
    o, lse = dta.attn_merge(o_parts, l_parts)
    torch.cuda.synchronize()
    del o_parts, l_parts
    _free()
    assert bool((o == 2.5).all())
    assert float((lse - math.log(4.0)).abs().max()) < 1e-6


def test_fp8_quant_past_2_31_elements():
    """Per-tensor E4M3 of 2^31 + 1000 bf16 values, zero but for three planted
    ones: amax = 896 at the last element gives scale 2; codes e4m3(x / 2):
    896 -> 448 (0x7E), -448 -> -224 (0xF6), 1.5 -> 0.75 (0x34)."""
    n = TWO31 + 1000
    _case("fp8_quant_per_tensor large", n=n)
    x = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    x[5] = -448.0
    x[TWO31 + 3] = 1.5
    x[n - 1] = 896.0
    x8, descale = dta.fp8_quant_per_tensor(x)
    torch.cuda.synchronize()
    del x
    _free()
    assert float(descale) == 2.0
    assert int(x8[n - 1]) == 0x7E and int(x8[5]) == 0xF6 and int(x8[TWO31 + 3]) == 0x34
    assert int(x8.count_nonzero()) == 3


@pytest.mark.parametrize("fn", ["residual_diff", "residual_diff_noalloc"])
def test_residual_diff_past_2_31_elements(fn):
    """b = 1 everywhere, a = 1 except its last 1000 elements, which are 3:
    sum|a - b| / sum|b| = 2000 / n exactly (every partial sum is an exact
    integer in float32 and float64)."""
    n = TWO31 + 77
    _case(fn + " large", n=n)
    b = torch.ones(n, dtype=torch.bfloat16, device=DEV)
    a = torch.ones_like(b)
    a[n - 1000:] = 3.0
    out = torch.empty((), dtype=torch.float32, device=DEV)
    if fn == "residual_diff":
        dta.residual_diff(a, b, out=out)
    else:
        dta.residual_diff_noalloc(a, b, out)
    torch.cuda.synchronize()
    del a, b
    _free()
    want = 2000.0 / n
    assert abs(float(out) - want) <= 1e-6 * want, (float(out), want)


def test_seq_concat_rows_past_2_31_elements():
    """Two token parts of 2^23 + 3 and 2^23 + 9 rows (D = 128) into one
    [1, 1, rows, 128] tensor of more than 2^31 elements: every row of part p
    holds p + 1."""
    lens = [(1 << 23) + 3, (1 << 23) + 9]
    D = 128
    assert sum(lens) * D > TWO31
    _case("seq_concat large", lens=lens, D=D)
    parts = torch.empty((sum(lens) * D,), dtype=torch.bfloat16, device=DEV)
    parts[:lens[0] * D].fill_(1.0)
    parts[lens[0] * D:].fill_(2.0)
    out = dta.seq_concat(parts, lens, B=1, H=1, D=D)
    torch.cuda.synchronize()
    del parts
    _free()
    out = out.view(sum(lens), D)
    assert bool((out[:lens[0]] == 1.0).all()) and bool((out[lens[0]:] == 2.0).all())
