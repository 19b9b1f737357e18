"""residual_diff_noalloc (the entry point for callers that cannot allocate)
through the C ABI against residual_diff and the oracle: two calls in a row
on the library's shared scratch, the second with a smaller input."""

import ctypes

import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
from diffusion_transformer_attention_flash_amd import _lib
import oracle
import workloads
from helpers import RESIDUAL_REL

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _call(fn, *args):
    st = fn(*args)
    assert st == _lib.DTA_OK, _lib.lib().dta_status_str(st).decode()


def test_noalloc_matches_residual_diff_twice_second_smaller():
    lib = _lib.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws = dta.workspace(DEV)
    cases = [workloads.residual_pair(5, (1, 4608, 3072), 0.08, device=DEV),   # FLUX residual
             workloads.residual_pair(9, (1_000_003,), 0.3, device=DEV)]      # smaller, ragged
    for i, (a, b) in enumerate(cases):
        print("CASE residual_diff_noalloc call %d, n=%d" % (i, a.numel()), flush=True)
        out_s = torch.full((), float("nan"), dtype=torch.float32, device=DEV)
        out_w = torch.full((), float("nan"), dtype=torch.float32, device=DEV)
        p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        _call(lib.residual_diff_noalloc, p(a), p(b), a.numel(), p(out_s), stream)
        _call(lib.residual_diff, p(a), p(b), a.numel(), p(out_w), p(ws), stream)
        torch.cuda.synchronize()
        got, want = out_s.item(), out_w.item()
        ref = oracle.residual_diff(a.cpu(), b.cpu())
        print("  noalloc %.9g  workspace %.9g  oracle %.9g" % (got, want, ref))
        assert got == want                                   # same kernel, same order
        assert abs(got - ref) <= RESIDUAL_REL * abs(ref)


def test_noalloc_binding_and_repeats():
    a, b = workloads.residual_pair(11, (3, 77, 1001), 0.05, device=DEV)
    print("CASE residual_diff_noalloc binding, n=%d" % a.numel(), flush=True)
    out = torch.empty((), dtype=torch.float32, device=DEV)
    vals = []
    for _ in range(5):
        dta.residual_diff_noalloc(a, b, out)
        vals.append(out.clone())
    torch.cuda.synchronize()
    assert all(v.item() == vals[0].item() for v in vals)
    assert vals[0].item() == dta.residual_diff(a, b).item()
