"""One GPU's share of the HunyuanVideo attention (B=1, H=24, N=119 056,
D=128) spread over 8 GPUs, at the share's real shape, through the calls a
rank makes. No collective runs: the buffers an exchange would deliver are
built in place from the full tensors.

* Ulysses (Context parallelism guide, Ulysses Attention): the all-to-all
  delivers this GPU's 3 heads of every token shard, packed shard after
  shard. seq_concat joins them, attn_fwd runs over all 119 056 tokens of
  the 3 heads, and seq_split cuts O back into token shards for the return
  exchange.
* Ring (same guide, Ring Attention): a rank keeps its 14 882 query rows of
  all 24 heads and folds the 8 K/V shards in turn: attn_fwd on the first,
  attn_fwd_accum on each of the other 7.

The layout steps must be exact permutations (bit for bit); the attention is
compared with the float64 oracle on seeded rows of every head."""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
import oracle
import workloads
from helpers import assert_bf16_attention

pytestmark = pytest.mark.gpu
DEV = "cuda"
P = 8


@pytest.fixture(scope="module")
def video():
    c = workloads.CONFIGS["hunyuan_720p_129f"]
    print("CASE share inputs hunyuan_720p_129f", flush=True)
    q, k, v = workloads.workload_qkv("hunyuan_720p_129f", device=DEV)
    return c, q, k, v


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_ulysses_share(video):
    c, q, k, v = video
    H, N, D = c["H"], c["N"], c["D"]
    hs, n = H // P, N // P
    gpu = 5                                   # holds heads 15, 16, 17
    h0 = gpu * hs
    print("CASE ulysses share: heads %d..%d of %d, N=%d" % (h0, h0 + hs - 1, H, N), flush=True)
    lens = [n] * P
    recv = [torch.cat([t[:, h0:h0 + hs, r * n:(r + 1) * n].reshape(-1) for r in range(P)])
            for t in (q, k, v)]
    qs, ks, vs = (dta.seq_concat(b, lens, 1, hs, D) for b in recv)
    for t, full in zip((qs, ks, vs), (q, k, v)):
        assert _same(t, full[:, h0:h0 + hs])
    scale = D ** -0.5
    o, lse = dta.attn_fwd(qs, ks, vs, scale)
    send = dta.seq_split(o, lens)
    torch.cuda.synchronize()
    for r in range(P):
        part = send[r * hs * n * D:(r + 1) * hs * n * D].view(1, hs, n, D)
        assert _same(part, o[:, :, r * n:(r + 1) * n])
    rows = workloads.sample_rows_per_head(c["config"], N, hs, c["sample_rows"], c["n_text"])
    for h in range(hs):
        rt = torch.from_numpy(rows[h]).to(DEV)
        o_ref, l_ref = oracle.attention(qs[:, h:h + 1, rt].cpu(), ks[:, h:h + 1].cpu(),
                                        vs[:, h:h + 1].cpu(), scale)
        assert_bf16_attention(o[:, h:h + 1, rt], lse[:, h:h + 1, rt], o_ref, l_ref,
                              "ulysses share, head %d" % (h0 + h))


def test_ring_share(video):
    c, q, k, v = video
    H, N, D = c["H"], c["N"], c["D"]
    n = N // P
    rank = 3
    print("CASE ring share: rank %d, rows %d..%d, %d K/V shards" % (rank, rank * n,
                                                                    (rank + 1) * n - 1, P),
          flush=True)
    scale = D ** -0.5
    qr = q[:, :, rank * n:(rank + 1) * n].contiguous()
    shards = workloads.split_kv(k, v, [n] * P)
    # The ring delivers the shards starting with the rank's own.
    order = [(rank + s) % P for s in range(P)]
    o, lse = dta.attn_fwd(qr, shards[order[0]][0], shards[order[0]][1], scale)
    for r in order[1:]:
        dta.attn_fwd_accum(qr, shards[r][0], shards[r][1], o, lse, scale)
    # All rows against one attn_fwd over the whole K/V (the same kernel's
    # single pass; the ring adds one bf16 rounding of O per step).
    o_full, l_full = dta.attn_fwd(qr, k, v, scale)
    torch.cuda.synchronize()
    assert_bf16_attention(o, lse, o_full, l_full, "ring share against one pass (all rows)")
    rows = workloads.sample_rows_per_head(c["config"], n, H, 32)
    for h in range(H):
        rt = torch.from_numpy(rows[h]).to(DEV)
        o_ref, l_ref = oracle.attention(qr[:, h:h + 1, rt].cpu(), k[:, h:h + 1].cpu(),
                                        v[:, h:h + 1].cpu(), scale)
        assert_bf16_attention(o[:, h:h + 1, rt], lse[:, h:h + 1, rt], o_ref, l_ref,
                              "ring share, head %d" % h)
    assert np.isfinite(lse.cpu().numpy()).all()
