"""GPU parity of residual_diff and fp8_quant_per_tensor against the oracle."""

import math

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
import oracle
import workloads
from helpers import RESIDUAL_REL

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rd(a, b):
    out = dta.residual_diff(a, b)
    torch.cuda.synchronize()
    return float(out.item())


def test_residual_diff_flux_residual_shape():
    c = workloads.CONFIGS["flux_1024_fp8"]
    print("CASE residual", c["residual_shape"], flush=True)
    a, b = workloads.residual_pair(c["config"], c["residual_shape"], c["residual_noise"], device=DEV)
    got = _rd(a, b)
    ref = oracle.residual_diff(a.cpu(), b.cpu())
    assert abs(got - ref) / ref <= RESIDUAL_REL, (got, ref)
    # bitwise reproducible
    assert _rd(a, b) == got


@pytest.mark.parametrize("n", [1, 7, 8, 9, 13, 4095, 4096 * 8 + 3, 1 << 20, 5_000_001])
def test_residual_diff_sizes(n):
    print("CASE residual n=%d" % n, flush=True)
    g = torch.Generator().manual_seed(n)
    b = torch.randn(n, generator=g).to(torch.bfloat16)
    a = (b.float() + 0.3 * torch.randn(n, generator=g)).to(torch.bfloat16)
    got = _rd(a.to(DEV), b.to(DEV))
    ref = oracle.residual_diff(a, b)
    assert abs(got - ref) <= RESIDUAL_REL * abs(ref), (got, ref)


def test_residual_diff_closed_forms():
    print("CASE residual closed forms", flush=True)
    b = torch.randn(123457, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    assert _rd(b, b) == 0.0
    assert _rd((2 * b.float()).to(torch.bfloat16), b) == pytest.approx(1.0, rel=1e-6)
    assert _rd(torch.zeros_like(b), b) == pytest.approx(1.0, rel=1e-6)
    assert _rd(-b, b) == pytest.approx(2.0, rel=1e-6)
    z = torch.zeros(100, dtype=torch.bfloat16, device=DEV)
    assert _rd(torch.ones_like(z), z) == math.inf
    assert math.isnan(_rd(z, z))


@pytest.mark.parametrize("shape", [(1, 24, 4608, 128), (3, 5, 64), (1000003,), (7,)])
def test_fp8_quant_bit_exact(shape):
    print("CASE quant", shape, flush=True)
    g = torch.Generator().manual_seed(sum(shape))
    x = (torch.randn(shape, generator=g) * 3).to(torch.bfloat16)
    x8, ds = dta.fp8_quant_per_tensor(x.to(DEV))
    torch.cuda.synchronize()
    codes, s = oracle.quant_per_tensor(x)
    assert float(ds.item()) == s
    got = x8.cpu().numpy()
    mism = int((got != codes).sum())
    assert mism == 0, "%d of %d codes differ" % (mism, codes.size)


def test_fp8_quant_zero_tensor_and_repeat():
    print("CASE quant zero", flush=True)
    z = torch.zeros(1000, dtype=torch.bfloat16, device=DEV)
    x8, ds = dta.fp8_quant_per_tensor(z)
    torch.cuda.synchronize()
    assert float(ds.item()) == 1.0 and int(x8.sum().item()) == 0
    # the workspace is re-armed: a second, different tensor quantises correctly
    x = torch.linspace(-3, 5, 999).to(torch.bfloat16)
    x8, ds = dta.fp8_quant_per_tensor(x.to(DEV))
    torch.cuda.synchronize()
    codes, s = oracle.quant_per_tensor(x)
    assert float(ds.item()) == s and (x8.cpu().numpy() == codes).all()


@pytest.mark.parametrize("sizes", [[(1000003,), (7,), (3, 5, 64)], [(4097,)],
                                   [(9,), (8,), (33, 17), (1, 2, 300, 128)]])
def test_fp8_quant_multi_bit_exact(sizes):
    """fp8_quant_per_tensor_multi gives every tensor the oracle's codes and
    scale, as fp8_quant_per_tensor does, whatever the mix of sizes (ragged
    tails, one tensor, four tensors, one all-zero tensor)."""
    print("CASE quant multi", sizes, flush=True)
    g = torch.Generator().manual_seed(len(sizes) * 100 + sum(len(s) for s in sizes))
    xs = [(torch.randn(s, generator=g) * (3.0 ** i)).to(torch.bfloat16) for i, s in enumerate(sizes)]
    if len(xs) == 4:
        xs[1] = torch.zeros(sizes[1], dtype=torch.bfloat16)
    x8s, ds = dta.fp8_quant_per_tensor_multi([x.to(DEV) for x in xs])
    torch.cuda.synchronize()
    for i, x in enumerate(xs):
        codes, s = oracle.quant_per_tensor(x)
        assert float(ds[i].item()) == s, i
        got = x8s[i].cpu().numpy()
        mism = int((got != codes).sum())
        assert mism == 0, "tensor %d: %d of %d codes differ" % (i, mism, codes.size)


def test_fp8_quant_multi_flux_qkv_matches_single():
    """Q, K and V of the FLUX shape in one call: bitwise what three single
    calls give."""
    print("CASE quant multi flux", flush=True)
    q, k, v = workloads.workload_qkv("flux_1024", device=DEV)
    x8s, ds = dta.fp8_quant_per_tensor_multi([q, k, v])
    singles = [dta.fp8_quant_per_tensor(t) for t in (q, k, v)]
    torch.cuda.synchronize()
    for i, (x8, d) in enumerate(singles):
        assert torch.equal(x8s[i], x8), i
        assert float(ds[i].item()) == float(d.item()), i


def test_reductions_on_two_streams():
    """The binding gives each (device, stream) its own reduction workspace, so
    residual_diff and the per-tensor quantiser issued on two streams at once
    give the results of calls on one stream, bit for bit."""
    print("CASE reductions on two streams", flush=True)
    c = workloads.CONFIGS["flux_1024_fp8"]
    a1, b1 = workloads.residual_pair(c["config"], c["residual_shape"], c["residual_noise"], device=DEV)
    a2, b2 = workloads.residual_pair(c["config"] + 1, (1, 1000, 3072), 0.5, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(3)
    x = torch.randn(1 << 22, generator=g, device=DEV).to(torch.bfloat16)
    r1, r2 = dta.residual_diff(a1, b1).clone(), dta.residual_diff(a2, b2).clone()
    x8, s = dta.fp8_quant_per_tensor(x)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        ws1 = dta.workspace(DEV)
    with torch.cuda.stream(s2):
        ws2 = dta.workspace(DEV)
    assert ws1.data_ptr() != ws2.data_ptr()
    got = []
    for _ in range(10):
        with torch.cuda.stream(s1):
            got.append(("r1", dta.residual_diff(a1, b1)))
            got.append(("q", dta.fp8_quant_per_tensor(x)))
        with torch.cuda.stream(s2):
            got.append(("r2", dta.residual_diff(a2, b2)))
    torch.cuda.synchronize()
    assert r1.item() != r2.item()
    for what, val in got:
        if what == "q":
            assert torch.equal(val[0], x8) and torch.equal(val[1], s)
        else:
            assert torch.equal(val, r1 if what == "r1" else r2), what


def test_residual_diff_last_workgroup_finish_repeats():
    """One launch per call: the workgroup that arrives last sums every
    partial. Fifty calls in a row (interleaved with per-tensor quantisations
    that share the workspace) give the same bits and agree with the oracle,
    and the workspace's arrival counter is back at zero after them."""
    print("CASE residual_diff repeated, shared workspace", flush=True)
    import diffusion_transformer_attention_flash_amd._lib as L
    a, b = workloads.residual_pair(5, (1, 4608, 3072), 0.08, device=DEV)
    x = torch.randn(3, 1000, 77, device=DEV).to(torch.bfloat16)
    outs = []
    for i in range(50):
        outs.append(dta.residual_diff(a, b).clone())
        if i % 7 == 3:
            dta.fp8_quant_per_tensor(x)
    torch.cuda.synchronize()
    first = outs[0].item()
    assert all(o.item() == first for o in outs) and math.isfinite(first)
    ref = oracle.residual_diff(a.cpu(), b.cpu())
    assert abs(first - ref) <= RESIDUAL_REL * ref
    # The workspace holds 16 KB of partials, then the arrival counters (a top
    # counter and one per group of workgroups, 256 bytes apart): all zero.
    ws = dta.workspace(DEV)
    n_ws = int(L.lib().dta_ws_bytes())
    assert n_ws > 16384
    assert int(ws[16384:n_ws].count_nonzero().item()) == 0
