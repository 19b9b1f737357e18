"""GPU parity of the fused ring step (attn_fwd_accum) and the pairwise
in-place merge (attn_merge_into), through the C ABI, against the oracle."""

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


def _ring(q, k, v, scale, lens, first="attn_fwd"):
    """Fold the K/V chunks in order into one running (o, lse)."""
    B, H, Nq, D = q.shape
    chunks = workloads.split_kv(k, v, lens)
    if first == "attn_fwd":
        o, lse = dta.attn_fwd(q, chunks[0][0], chunks[0][1], scale)
        rest = chunks[1:]
    else:
        # start from "nothing seen": LSE -inf, O garbage (NaN) that must be ignored
        o = torch.full((B, H, Nq, D), float("nan"), dtype=torch.bfloat16, device=q.device)
        lse = torch.full((B, H, Nq), -math.inf, dtype=torch.float32, device=q.device)
        rest = chunks
    for kc, vc in rest:
        dta.attn_fwd_accum(q, kc, vc, o, lse, scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("first", ["attn_fwd", "empty"])
def test_tiny_ring_matches_full_attention(first):
    c = workloads.CONFIGS["tiny"]
    print("CASE tiny ring first=%s" % first, flush=True)
    q, k, v = workloads.workload_qkv("tiny", device=DEV)
    scale = 1.0 / math.sqrt(c["D"])
    o, lse = _ring(q, k, v, scale, c["chunks"], first)
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    assert_bf16_attention(o, lse, o_ref, lse_ref, "tiny ring (%s)" % first)


@pytest.mark.parametrize("D,lens", [(64, [1, 63, 64, 130]), (128, [200, 7, 65, 300]),
                                    (128, [64]), (64, [5, 5, 5])])
def test_ring_ragged_chunks(D, lens):
    """Chunks with ragged tails (1, 5, 7, 63 ... keys) and a single-chunk ring."""
    print("CASE ring D=%d lens=%s" % (D, lens), flush=True)
    B, H, Nq, Nkv = 1, 2, 300, sum(lens)
    q, k, v = workloads.make_qkv(1, B, H, Nq, Nkv, D, device=DEV)
    scale = D ** -0.5
    o, lse = _ring(q, k, v, scale, lens, "empty")
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    assert_bf16_attention(o, lse, o_ref, lse_ref, "ring D=%d" % D)


def test_flux_ring_eight_uneven_chunks():
    """The 8-chunk FLUX ring at full size, every row; and the fused step
    against attn_fwd + the oracle's two-part merge of the same running state."""
    c = workloads.CONFIGS["flux_1024_chunked"]
    lens = workloads.chunk_lengths(c["config"], c["N"], c["n_chunks"], c["min_chunk"])
    print("CASE flux ring", lens, flush=True)
    q, k, v = workloads.workload_qkv("flux_1024_chunked", device=DEV)
    scale = c["D"] ** -0.5
    o, lse = _ring(q, k, v, scale, lens)
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    assert_bf16_attention(o, lse, o_ref, lse_ref, "flux ring (all rows)")

    # one fused step in isolation: state after 7 chunks, then chunk 8
    o7, l7 = _ring(q, k[:, :, :sum(lens[:7])], v[:, :, :sum(lens[:7])], scale, lens[:7])
    o7_before, l7_before = o7.clone(), l7.clone()
    kc, vc = workloads.split_kv(k, v, lens)[7]
    oc, lc = dta.attn_fwd(q, kc, vc, scale)
    dta.attn_fwd_accum(q, kc, vc, o7, l7, scale)
    torch.cuda.synchronize()
    om, lm = oracle.merge(torch.stack([o7_before.cpu(), oc.cpu()]),
                          torch.stack([l7_before.cpu(), lc.cpu()]))
    # The fused step merges the unrounded chunk output, the oracle gets
    # attn_fwd's bf16-rounded one: they differ by at most the chunk's merge
    # weight f_c times one bf16 ulp of O_c, plus one ulp of the merged O.
    f_c = 1.0 / (1.0 + np.exp(to64(l7_before) - to64(lc)))[..., None]
    d = np.abs(to64(o7) - om)
    tol = 2.0 ** -8 * (f_c * np.abs(to64(oc)) + np.abs(om)) + 1e-6
    assert (d <= tol).all(), "fused step differs from merge(state, attn_fwd) by %.3e" % d.max()
    assert np.abs(to64(l7) - lm).max() < 1e-4


@pytest.mark.parametrize("D", [64, 128])
def test_merge_into_random_partials(D):
    print("CASE merge_into D=%d" % D, flush=True)
    g = torch.Generator().manual_seed(700 + D)
    B, H, Nq = 2, 3, 91
    oa = torch.randn((B, H, Nq, D), generator=g).to(torch.bfloat16)
    ob = torch.randn((B, H, Nq, D), generator=g).to(torch.bfloat16)
    la = (torch.randn((B, H, Nq), generator=g) * 5).to(torch.float32)
    lb = (torch.randn((B, H, Nq), generator=g) * 5).to(torch.float32)
    la[0, 0, :10] = -math.inf                 # running state empty: take the part
    oa[0, 0, :10] = float("nan")              # ... and never touch its O
    lb[1, 2, 20:30] = -math.inf               # the part saw nothing
    ob[1, 2, 20:30] = float("nan")
    la[1, 1, 40] = lb[1, 1, 40] = -math.inf   # neither saw anything
    # The oracle sees zeros where the kernel sees NaN: a weight-0 part's O must
    # not matter, so both are the same merge.
    om, lm = oracle.merge(torch.stack([torch.nan_to_num(oa, nan=0.0), torch.nan_to_num(ob, nan=0.0)]),
                          torch.stack([la, lb]))
    o, lse = oa.to(DEV), la.to(DEV)
    dta.attn_merge_into(o, lse, ob.to(DEV), lb.to(DEV))
    torch.cuda.synchronize()
    fin = np.isfinite(lm)
    assert np.isfinite(to64(o)).all()
    d = np.abs(to64(o) - om)
    assert (d <= np.maximum(np.abs(om), 2.0 ** -126) * 2.0 ** -8 + 1e-6).all()
    np.testing.assert_allclose(to64(lse)[fin], lm[fin], rtol=0, atol=1e-5)
    assert (to64(lse)[~fin] == -np.inf).all() and (to64(o)[~fin] == 0).all()
