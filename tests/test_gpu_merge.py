"""GPU parity of the chunked ring-step path: attn_fwd per K/V chunk + attn_merge."""

import math

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
import oracle
import workloads
from helpers import assert_bf16_attention, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _chunked(q, k, v, scale, lens):
    n = len(lens)
    B, H, Nq, D = q.shape
    o_parts = torch.empty((n, B, H, Nq, D), dtype=torch.bfloat16, device=q.device)
    l_parts = torch.empty((n, B, H, Nq), dtype=torch.float32, device=q.device)
    for i, (kc, vc) in enumerate(workloads.split_kv(k, v, lens)):
        dta.attn_fwd(q, kc, vc, scale, o=o_parts[i], lse=l_parts[i])
    o, lse = dta.attn_merge(o_parts, l_parts)
    torch.cuda.synchronize()
    return o, lse, o_parts, l_parts


def test_tiny_four_chunks():
    c = workloads.CONFIGS["tiny"]
    print("CASE tiny 4x64 chunks", flush=True)
    q, k, v = workloads.workload_qkv("tiny", device=DEV)
    scale = 1.0 / math.sqrt(c["D"])
    o, lse, _, _ = _chunked(q, k, v, scale, c["chunks"])
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    assert_bf16_attention(o, lse, o_ref, lse_ref, "tiny chunked")
    o1, l1 = dta.attn_fwd(q, k, v, scale)
    torch.cuda.synchronize()
    # chunked and unchunked agree to bf16 output rounding
    assert np.abs(to64(o) - to64(o1)).max() < 2e-3


def test_flux_eight_uneven_chunks():
    c = workloads.CONFIGS["flux_1024_chunked"]
    lens = workloads.chunk_lengths(c["config"], c["N"], c["n_chunks"], c["min_chunk"])
    print("CASE flux_1024_chunked", lens, flush=True)
    q, k, v = workloads.workload_qkv("flux_1024_chunked", device=DEV)
    scale = c["D"] ** -0.5
    o, lse, o_parts, l_parts = _chunked(q, k, v, scale, lens)
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    assert_bf16_attention(o, lse, o_ref, lse_ref, "flux chunked (all rows)")
    # merge in isolation: the oracle's merge of the GPU's own partials, every row
    om, lm = oracle.merge(o_parts.cpu(), l_parts.cpu())
    d_o = np.abs(to64(o) - om)
    ulp = np.maximum(np.abs(om), 2.0 ** -126) * 2.0 ** -8     # one bf16 ulp (upper bound)
    assert (d_o <= ulp + 1e-6).all(), "merge differs from oracle merge by > 1 bf16 ulp"
    assert np.abs(to64(lse) - lm).max() < 1e-5


# Every instantiated partial count (1..8, one kernel each) at both head dims,
# and the generic kernel (more than 8 partials).
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n_parts", [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 13])
def test_merge_random_partials(n_parts, D):
    print("CASE merge n=%d D=%d" % (n_parts, D), flush=True)
    g = torch.Generator().manual_seed(100 + n_parts + D)
    B, H, Nq = 2, 3, 77
    o_parts = torch.randn((n_parts, B, H, Nq, D), generator=g).to(torch.bfloat16)
    l_parts = (torch.randn((n_parts, B, H, Nq), generator=g) * 5).to(torch.float32)
    o_dev = o_parts.clone()
    if n_parts >= 2:
        l_parts[1, 0, 0, :] = -math.inf            # a chunk that saw nothing
        o_dev[1, 0, 0, :] = math.nan               # its O is garbage: weight 0 must not read it
        o_parts[1, 0, 0, :] = 0.0                  # (the oracle's sum would take 0 * NaN = NaN)
    l_parts[:, 1, 2, 5] = -math.inf                # a row with nothing at all
    o_dev[:, 1, 2, 5] = math.nan
    o_parts[:, 1, 2, 5] = 0.0
    o, lse = dta.attn_merge(o_dev.to(DEV), l_parts.to(DEV))
    torch.cuda.synchronize()
    om, lm = oracle.merge(o_parts, l_parts)
    fin = np.isfinite(lm)
    d_o = np.abs(to64(o) - om)
    ulp = np.maximum(np.abs(om), 2.0 ** -126) * 2.0 ** -8     # one bf16 ulp (upper bound)
    assert (d_o <= ulp + 1e-6).all(), "merge differs from oracle merge by > 1 bf16 ulp"
    np.testing.assert_allclose(to64(lse)[fin], lm[fin], rtol=0, atol=1e-5)
    assert (to64(lse)[~fin] == -np.inf).all()
    assert (to64(o)[~fin] == 0).all()
