"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This module holds input generation only -- none of the attention, merge,
quantisation or residual arithmetic. The HIP path and the CPU oracle both
consume exactly the tensors made here.

The shapes stand in for the attention activations of the two diffusion
transformers the ParaAttention guide benchmarks (no weights or prompts are
available, so values are random):

* FLUX.1-dev at 1024x1024 (ParaAttention guide, sections "First Block Cache"
  and "Benchmarks"): 64x64 = 4096 image tokens after 2x2 patching of the
  128x128 latent, plus 512 text tokens -> N = 4608, 24 heads of 128.
* HunyuanVideo at 720x1280, 129 frames (same guide): 33 latent frames of
  45x80 patches = 118800 video tokens plus 256 text tokens -> N = 119056,
  24 heads of 128.

Recipe (all seeded; one torch.Generator per tensor):

* Q, K ~ N(0, 1) in float32, then RMS-normalised per (b, h, token) row over D
  (x / sqrt(mean x^2 + 1e-6), no affine weight -- the QK-norm these models
  apply before attention), then rounded to bf16 (round-to-nearest-even).
* V ~ N(0, 1) float32 -> bf16.
* The tiny case draws Q, K, V i.i.d. N(0, 1) float32 without QK-norm and
  rounds to bf16 for both sides.
* Seeds: 20000 + 100 * config + slot, slot Q=0, K=1, V=2, noise=3; chunk
  lengths use numpy default_rng(seed slot 4), sampled rows slot 5, the
  residual pair's b slot 6 and its noise slot 3.
"""

import numpy as np
import torch

# name -> shape and options. "config" is the index used in the seeds.
CONFIGS = {
    "tiny": dict(config=1, B=1, H=2, N=256, D=64, qknorm=False,
                 chunks=[64, 64, 64, 64], n_text=0),
    "flux_1024": dict(config=2, B=1, H=24, N=4608, D=128, qknorm=True,
                      n_text=512),
    "flux_1024_chunked": dict(config=3, B=1, H=24, N=4608, D=128,
                              qknorm=True, n_chunks=8, min_chunk=64,
                              n_text=512),
    "hunyuan_720p_129f": dict(config=4, B=1, H=24, N=119056, D=128,
                              qknorm=True, sample_rows=256, n_text=256),
    "flux_1024_fp8": dict(config=5, B=1, H=24, N=4608, D=128, qknorm=True,
                          n_text=512, residual_shape=(1, 4608, 3072),
                          residual_noise=0.08),
}

SLOT_Q, SLOT_K, SLOT_V, SLOT_NOISE, SLOT_CHUNKS, SLOT_ROWS, SLOT_RES = 0, 1, 2, 3, 4, 5, 6


def seed_of(config, slot):
    return 20000 + 100 * int(config) + int(slot)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, seed, device):
    return torch.randn(*shape, generator=_gen(device, seed), device=device,
                       dtype=torch.float32)


def _rms_rows(x):
    # QK-norm of the input recipe (not part of the attention being tested).
    return x * torch.rsqrt(x.pow(2).mean(dim=-1, keepdim=True) + 1e-6)


def make_qkv(config, B, H, Nq, Nkv, D, qknorm=True, device="cpu",
             q_gain=1.0, dtype=torch.bfloat16):
    """Seeded Q [B,H,Nq,D], K, V [B,H,Nkv,D] in ``dtype`` on ``device``.

    ``q_gain`` multiplies Q in float32 before the bf16 rounding; a gain of 4
    makes the logits' spread ~4x wider ("peaked" rows whose O is O(1)).
    """
    q = _normal((B, H, Nq, D), seed_of(config, SLOT_Q), device)
    k = _normal((B, H, Nkv, D), seed_of(config, SLOT_K), device)
    if qknorm:
        q = _rms_rows(q)
        k = _rms_rows(k)
    if q_gain != 1.0:
        q = q * float(q_gain)
    q = q.to(dtype)
    k = k.to(dtype)
    v = _normal((B, H, Nkv, D), seed_of(config, SLOT_V), device).to(dtype)
    return q, k, v


def workload_qkv(name, device="cpu"):
    c = CONFIGS[name]
    return make_qkv(c["config"], c["B"], c["H"], c["N"], c["N"], c["D"],
                    qknorm=c["qknorm"], device=device)


def chunk_lengths(config, n_total, n_chunks, min_len=64):
    """Seeded uneven contiguous chunk lengths, each >= min_len, summing to n_total."""
    if n_chunks * min_len > n_total:
        raise ValueError("chunks cannot all reach min_len")
    rng = np.random.default_rng(seed_of(config, SLOT_CHUNKS))
    extra = rng.multinomial(n_total - n_chunks * min_len,
                            [1.0 / n_chunks] * n_chunks)
    lens = [int(min_len + e) for e in extra]
    assert sum(lens) == n_total
    return lens


def sample_rows(config, n, count=256, n_text=0, tile=64):
    """Seeded query rows: the edge rows forced in, the rest drawn uniformly.

    Forced rows: the first, the text/video boundary pair, the last, and the
    first row of the partial last tile (or of the last full tile).
    """
    forced = [0, n - 1]
    if 0 < n_text < n:
        forced += [n_text - 1, n_text]
    forced.append(n - (n % tile) if n % tile else max(n - tile, 0))
    forced = sorted(set(int(r) for r in forced if 0 <= r < n))
    rng = np.random.default_rng(seed_of(config, SLOT_ROWS))
    pool = np.setdiff1d(np.arange(n), np.asarray(forced))
    k = max(0, min(count - len(forced), pool.size))
    drawn = rng.choice(pool, size=k, replace=False)
    return np.sort(np.concatenate([np.asarray(forced), drawn]).astype(np.int64))


def sample_rows_per_head(config, n, heads, count=256, n_text=0, block=32, tile=64):
    """Seeded query rows for each head: an int64 array [heads, count], each
    head's rows sorted and distinct.

    Every head gets the forced edge rows of ``sample_rows``. The ``block``-row
    blocks of the sequence are dealt round-robin to the heads (block b to
    head b % heads) and each head draws one row inside each of its blocks, so
    that across the heads every block of ``block`` consecutive query rows is
    compared at least once when ``count`` leaves room for it (otherwise a
    seeded subset of the head's blocks); the remaining rows are drawn
    uniformly from the rest. One random stream per head, seeded by the
    config's rows slot and the head index.
    """
    count = min(int(count), int(n))
    forced = [0, n - 1]
    if 0 < n_text < n:
        forced += [n_text - 1, n_text]
    forced.append(n - (n % tile) if n % tile else max(n - tile, 0))
    forced = sorted(set(int(r) for r in forced if 0 <= r < n))[:count]
    n_blocks = -(-int(n) // block)
    out = np.empty((heads, count), dtype=np.int64)
    for h in range(heads):
        rng = np.random.default_rng([seed_of(config, SLOT_ROWS), h])
        mine = np.arange(h, n_blocks, heads)
        room = count - len(forced)
        if mine.size > room:
            mine = np.sort(rng.choice(mine, size=room, replace=False))
        lo = mine * block
        hi = np.minimum(lo + block, n)
        picked = lo + (rng.random(mine.size) * (hi - lo)).astype(np.int64)
        chosen = np.union1d(np.asarray(forced, dtype=np.int64), picked)
        pool = np.setdiff1d(np.arange(n), chosen)
        extra = rng.choice(pool, size=count - chosen.size, replace=False)
        out[h] = np.sort(np.concatenate([chosen, extra]))
    return out


def residual_pair(config, shape, noise=0.08, device="cpu"):
    """b ~ N(0,1) -> bf16; a = bf16(float(b) + noise * N(0,1))."""
    b = _normal(shape, seed_of(config, SLOT_RES), device).to(torch.bfloat16)
    n = _normal(shape, seed_of(config, SLOT_NOISE), device)
    a = (b.to(torch.float32) + float(noise) * n).to(torch.bfloat16)
    return a, b


def split_kv(k, v, lens):
    """Contiguous copies of consecutive K/V slices along the token axis."""
    out, start = [], 0
    for n in lens:
        out.append((k[:, :, start:start + n].contiguous(),
                    v[:, :, start:start + n].contiguous()))
        start += n
    return out
