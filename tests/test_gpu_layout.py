"""GPU parity of the layout kernels (seq/head split and concat with uneven
and padded parts) through the C ABI: bit-exact against oracle.layout."""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_flash_amd as dta
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rand16(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16)


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy()


def _pack(parts):
    return torch.cat([p.reshape(-1) for p in parts])


@pytest.mark.parametrize("B,H,D,lens,pads", [
    (1, 24, 128, [576] * 8, None),                    # Ulysses share of the FLUX shape
    (2, 3, 64, [5, 0, 17, 1], [8, 3, 17, 4]),         # uneven, empty part, padding
    (1, 2, 40, [1], [9]),                             # Ring Anything pad of one shard
    (1, 3, 128, [7, 64, 65, 1, 200], None),
])
def test_seq_split_and_concat(B, H, D, lens, pads):
    print("CASE seq B=%d H=%d D=%d lens=%s pads=%s" % (B, H, D, lens, pads), flush=True)
    x = _rand16((B, H, sum(lens), D), 100 + D)
    parts = dta.seq_split(x.to(DEV), lens, pads)
    torch.cuda.synchronize()
    want = oracle.layout.seq_split(x.view(torch.int16).numpy(), lens, pads)
    assert np.array_equal(_bits(parts), np.concatenate([w.ravel() for w in want]))
    # concat of the GPU's parts (and of oracle parts holding garbage in the pad rows)
    pad_list = lens if pads is None else pads
    noisy = [torch.from_numpy(w.copy()) for w in want]
    for p, (n, pad) in enumerate(zip(lens, pad_list)):
        noisy[p][:, :, n:] = 12345                    # must never be read
    out = dta.seq_concat(_pack(noisy).view(torch.bfloat16).to(DEV), lens, B, H, D, padded=pads)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), x.view(torch.int16).numpy())


@pytest.mark.parametrize("B,N,D,heads", [
    (1, 4608, 128, [3] * 8),
    (2, 37, 64, [1, 4, 2]),
    (3, 5, 8, [2]),
])
def test_head_split_and_concat(B, N, D, heads):
    print("CASE head B=%d N=%d D=%d heads=%s" % (B, N, D, heads), flush=True)
    x = _rand16((B, sum(heads), N, D), 200 + N)
    parts = dta.head_split(x.to(DEV), heads)
    torch.cuda.synchronize()
    want = oracle.layout.head_split(x.view(torch.int16).numpy(), heads)
    assert np.array_equal(_bits(parts), np.concatenate([w.ravel() for w in want]))
    out = dta.head_concat(parts, heads, B, N, D)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), x.view(torch.int16).numpy())


def test_ulysses_round_trip_on_the_gpu():
    """Three ranks emulated on one GPU, uneven tokens and heads: the forward
    and backward Ulysses permutations reproduce global slicing exactly."""
    B, D = 1, 128
    n_rank, h_rank = [300, 17, 211], [5, 1, 2]
    N, H = sum(n_rank), sum(h_rank)
    X = _rand16((B, H, N, D), 7).to(DEV)
    toff = np.concatenate([[0], np.cumsum(n_rank)])
    hoff = np.concatenate([[0], np.cumsum(h_rank)])
    sent = []
    for r in range(3):
        buf = dta.head_split(X[:, :, toff[r]:toff[r + 1]].contiguous(), h_rank)
        sizes = [B * h * n_rank[r] * D for h in h_rank]
        sent.append(torch.split(buf, sizes))
    for r in range(3):
        recv = torch.cat([sent[s][r] for s in range(3)])          # all-to-all
        mine = dta.seq_concat(recv, n_rank, B, h_rank[r], D)
        torch.cuda.synchronize()
        assert torch.equal(mine, X[:, hoff[r]:hoff[r + 1]])
