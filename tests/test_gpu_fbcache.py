"""GPU parity of fbcache_step (First Block Cache decision + cached-residual
apply, on the device) through the C ABI, against oracle.fbcache_step."""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
import oracle
import workloads
from helpers import RESIDUAL_REL, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(n, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return ((torch.randn(n, generator=g) * scale).to(torch.bfloat16),
            (torch.randn(n, generator=g) * scale).to(torch.bfloat16))


def _run(r, rp, thr, hidden, cached):
    h = hidden.clone().to(DEV)
    diff, use = dta.fbcache_step(r.to(DEV), rp.to(DEV), thr, h, cached.to(DEV))
    torch.cuda.synchronize()
    return float(diff.item()), int(use.item()), h.cpu()


@pytest.mark.parametrize("thr", [0.12, 0.05])
def test_flux_residual_workload(thr):
    """The FLUX-shape residual pair (diff ~ 0.08) with the first block's hidden
    states of the same shape, at a threshold above and one below the diff."""
    c = workloads.CONFIGS["flux_1024_fp8"]
    print("CASE fbcache flux thr=%g" % thr, flush=True)
    r, rp = workloads.residual_pair(c["config"], c["residual_shape"], c["residual_noise"])
    hidden, cached = _pair(r.numel(), 31)
    hidden, cached = hidden.view(r.shape), cached.view(r.shape)
    d_gpu, use_gpu, h_gpu = _run(r, rp, thr, hidden, cached)
    d_ref, use_ref, h_ref = oracle.fbcache_step(r, rp, thr, hidden, cached)
    assert abs(d_gpu - d_ref) <= RESIDUAL_REL * d_ref
    assert use_gpu == int(use_ref) == int(thr > d_ref)
    assert np.array_equal(to64(h_gpu), h_ref)        # bit-exact bf16 sums (or untouched)


@pytest.mark.parametrize("n_hidden", [1, 7, 8, 13, 4096 + 5, 1_000_003])
def test_apply_bit_exact_ragged(n_hidden):
    print("CASE fbcache apply n=%d" % n_hidden, flush=True)
    r, rp = _pair(2048, 41)
    rp = (r.float() * 1.01).to(torch.bfloat16)      # diff ~ 0.01: reuse at 0.08
    hidden, cached = _pair(n_hidden, 43 + n_hidden, scale=3.0)
    cached[: min(5, n_hidden)] = torch.tensor([1e-30, -1e30, 0.0, -0.0, 65504.0][: min(5, n_hidden)]).to(torch.bfloat16)
    d_gpu, use_gpu, h_gpu = _run(r, rp, 0.08, hidden, cached)
    d_ref, use_ref, h_ref = oracle.fbcache_step(r, rp, 0.08, hidden, cached)
    assert use_gpu == 1 and use_ref
    assert np.array_equal(to64(h_gpu), h_ref)


def test_threshold_equal_to_diff_does_not_reuse():
    """Strict compare on the device's own float32 diff: thr = diff -> 0, the
    next float32 above it -> 1."""
    r, rp = _pair(100_000, 51)
    hidden, cached = _pair(1000, 52)
    d, _, _ = _run(r, rp, 0.5, hidden, cached)
    _, use_eq, h_eq = _run(r, rp, d, hidden, cached)
    assert use_eq == 0 and torch.equal(h_eq, hidden)
    up = float(np.nextafter(np.float32(d), np.float32(np.inf)))
    _, use_up, h_up = _run(r, rp, up, hidden, cached)
    assert use_up == 1 and not torch.equal(h_up, hidden)


def test_zero_previous_residual_never_reuses():
    hidden, cached = _pair(777, 61)
    z = torch.zeros(4096, dtype=torch.bfloat16)
    x, _ = _pair(4096, 62)
    d, use, h = _run(x, z, 1e30, hidden, cached)      # x / 0 = inf
    assert use == 0 and np.isinf(d) and torch.equal(h, hidden)
    d, use, h = _run(z, z, 1e30, hidden, cached)      # 0 / 0 = NaN
    assert use == 0 and np.isnan(d) and torch.equal(h, hidden)


def test_repeat_is_bitwise_identical_and_flag_consistent():
    r, rp = _pair(3_000_001, 71)
    hidden, cached = _pair(5000, 72)
    out = [_run(r, rp, 2.0, hidden, cached) for _ in range(3)]
    assert len({o[0] for o in out}) == 1
    assert all(o[1] == int(o[0] < 2.0) for o in out)
    assert all(torch.equal(o[2], out[0][2]) for o in out)
