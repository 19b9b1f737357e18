"""GPU parity of attn_fwd (bf16) against the float64 oracle, through the C ABI.

Every test prints what it runs before it runs it, so that a failure on the
GPU names its case.
"""

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


def _run(q, k, v, scale):
    o, lse = dta.attn_fwd(q, k, v, scale)
    torch.cuda.synchronize()
    return o, lse


def _case(name, **kw):
    print("CASE", name, kw, flush=True)


def test_tiny_config_all_rows():
    c = workloads.CONFIGS["tiny"]
    _case("tiny", **{k: c[k] for k in ("B", "H", "N", "D")})
    q, k, v = workloads.workload_qkv("tiny", device=DEV)
    scale = 1.0 / math.sqrt(c["D"])
    o, lse = _run(q, k, v, scale)
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    assert_bf16_attention(o, lse, o_ref, lse_ref, "tiny")
    # information only: error against the unrounded float32 inputs
    qf, kf, vf = workloads.make_qkv(1, 1, 2, 256, 256, 64, qknorm=False, dtype=torch.float32)
    o32, _ = oracle.attention(qf, kf, vf, scale)
    print("tiny vs unrounded fp32 inputs: O max-abs %.3e" % np.abs(to64(o) - o32).max())


@pytest.mark.parametrize("B,H,Nq,Nkv,D", [
    (1, 2, 300, 300, 128),       # ragged query and key tails, several tiles
    (2, 3, 129, 1000, 64),
    (1, 1, 1, 1, 128),           # one query, one key
    (1, 2, 33, 1, 64),
    (1, 1, 64, 15, 128), (1, 1, 64, 16, 128), (1, 1, 64, 63, 128),
    (1, 1, 64, 64, 128), (1, 1, 64, 65, 128), (1, 1, 64, 127, 128),
    (1, 1, 64, 129, 128),
    (1, 1, 31, 200, 64), (1, 1, 127, 200, 64), (1, 1, 129, 200, 64),
    (3, 2, 700, 517, 128),
])
def test_shapes_all_rows(B, H, Nq, Nkv, D):
    _case("shape", B=B, H=H, Nq=Nq, Nkv=Nkv, D=D)
    q, k, v = workloads.make_qkv(7, B, H, Nq, Nkv, D, qknorm=True, device=DEV)
    scale = D ** -0.5
    o, lse = _run(q, k, v, scale)
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    assert_bf16_attention(o, lse, o_ref, lse_ref, "shape")


@pytest.mark.parametrize("D", [64, 128])
def test_peaked_rows(D):
    # Q x4 before rounding: logits spread ~4x wider, O is O(1) and a broken
    # softmax cannot hide under the small random-input O.
    _case("peaked", D=D)
    q, k, v = workloads.make_qkv(11, 1, 4, 520, 777, D, qknorm=True, device=DEV, q_gain=4.0)
    o, lse = _run(q, k, v, D ** -0.5)
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), D ** -0.5)
    assert np.abs(o_ref).max() > 0.5
    assert_bf16_attention(o, lse, o_ref, lse_ref, "peaked")


@pytest.mark.parametrize("D", [64, 128])
def test_extreme_logits(D):
    """Q x64 before rounding: the logits spread over hundreds of units, every
    row's softmax is nearly one-hot, and the running max jumps between tiles
    by far more than the lazy-rescale slack (the rescale factor underflows
    to 0). The same attention as a fused ring over three chunks."""
    _case("extreme logits", D=D)
    q, k, v = workloads.make_qkv(13, 1, 2, 300, 1000, D, qknorm=True, device=DEV, q_gain=64.0)
    # A nearly one-hot row returns one V row, up to ~4.4 here, where one bf16
    # rounding alone is up to 1.6e-2; V / 4 (exact) keeps |O| near 1 so that
    # the absolute O gate measures the kernel, not the output format.
    v = v * 0.25
    scale = D ** -0.5
    o, lse = _run(q, k, v, scale)
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    assert np.abs(lse_ref).max() > 50
    assert_bf16_attention(o, lse, o_ref, lse_ref, "extreme")
    chunks = workloads.split_kv(k, v, [333, 1, 666])
    o_r, lse_r = dta.attn_fwd(q, chunks[0][0], chunks[0][1], scale)
    for kc, vc in chunks[1:]:
        dta.attn_fwd_accum(q, kc, vc, o_r, lse_r, scale)
    torch.cuda.synchronize()
    assert_bf16_attention(o_r, lse_r, o_ref, lse_ref, "extreme ring")


def test_closed_forms_on_gpu():
    _case("closed-forms")
    D, n = 128, 333
    q, k, v = workloads.make_qkv(13, 1, 2, 100, n, D, qknorm=True, device=DEV)
    # identical keys -> O = mean V, LSE = scale q.k + ln n
    k_same = k[:, :, :1].expand(-1, -1, n, -1).contiguous()
    o, lse = _run(q, k_same, v, D ** -0.5)
    o_ref, lse_ref = oracle.attention(q.cpu(), k_same.cpu(), v.cpu(), D ** -0.5)
    assert_bf16_attention(o, lse, o_ref, lse_ref, "identical-keys")
    mean_v = to64(v).mean(axis=2, keepdims=True)
    assert np.abs(to64(o) - mean_v).max() < 2e-3
    # constant V -> O = that constant
    v_c = torch.full_like(v, -0.75)
    o, _ = _run(q, k, v_c, D ** -0.5)
    assert np.abs(to64(o) + 0.75).max() < 4e-3
    # one key -> O = v0, LSE = scale q.k0
    o, lse = _run(q, k[:, :, :1].contiguous(), v[:, :, :1].contiguous(), D ** -0.5)
    assert np.abs(to64(o) - to64(v[:, :, :1])).max() < 4e-3
    # scale 0 -> uniform weights: O = mean V, LSE = ln n
    o, lse = _run(q, k, v, 0.0)
    assert np.abs(to64(o) - mean_v).max() < 2e-3
    assert np.abs(to64(lse) - math.log(n)).max() < 1e-4
    # permuting keys and values together leaves the result unchanged
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(3)).to(DEV)
    o1, l1 = _run(q, k, v, D ** -0.5)
    o2, l2 = _run(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), D ** -0.5)
    assert np.abs(to64(o1) - to64(o2)).max() < 2e-3
    assert np.abs(to64(l1) - to64(l2)).max() < 1e-4


def test_deterministic_and_guard_bands():
    _case("determinism+canary")
    B, H, Nq, Nkv, D = 1, 3, 450, 611, 128
    q, k, v = workloads.make_qkv(17, B, H, Nq, Nkv, D, device=DEV)
    pad = 4096
    o_buf = torch.full((pad + B * H * Nq * D + pad,), 12345, dtype=torch.int16, device=DEV)
    l_buf = torch.full((pad + B * H * Nq + pad,), 7.0, dtype=torch.float32, device=DEV)
    o = o_buf[pad:pad + B * H * Nq * D].view(torch.bfloat16).view(B, H, Nq, D)
    lse = l_buf[pad:pad + B * H * Nq].view(B, H, Nq)
    dta.attn_fwd(q, k, v, D ** -0.5, o=o, lse=lse)
    o2, l2 = dta.attn_fwd(q, k, v, D ** -0.5)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse, l2)
    assert bool((o_buf[:pad] == 12345).all()) and bool((o_buf[-pad:] == 12345).all())
    assert bool((l_buf[:pad] == 7.0).all()) and bool((l_buf[-pad:] == 7.0).all())


def test_flux_1024_all_rows():
    # The 4608-token FLUX.1-dev shape at the launch configuration the bench
    # times; every query row of every head against the oracle.
    c = workloads.CONFIGS["flux_1024"]
    _case("flux_1024", **{k: c[k] for k in ("B", "H", "N", "D")})
    q, k, v = workloads.workload_qkv("flux_1024", device=DEV)
    scale = c["D"] ** -0.5
    o, lse = _run(q, k, v, scale)
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale)
    assert_bf16_attention(o, lse, o_ref, lse_ref, "flux_1024 (all rows)")


def test_hunyuan_video_rows_per_head():
    # 119056 tokens: generated on the GPU; each head's 256 rows (forced edge
    # rows plus one row in each 32-row block dealt to that head, so the 24
    # heads together cover every 32-row block) and its K/V are copied back,
    # so the oracle sees exactly the bytes the kernel read.
    c = workloads.CONFIGS["hunyuan_720p_129f"]
    _case("hunyuan_720p_129f", **{k: c[k] for k in ("B", "H", "N", "D")})
    q, k, v = workloads.workload_qkv("hunyuan_720p_129f", device=DEV)
    scale = c["D"] ** -0.5
    o, lse = _run(q, k, v, scale)
    rows = workloads.sample_rows_per_head(c["config"], c["N"], c["H"], c["sample_rows"], c["n_text"])
    for h in range(c["H"]):
        rt = torch.from_numpy(rows[h]).to(DEV)
        o_ref, l_ref = oracle.attention(q[:, h:h + 1, rt].cpu(), k[:, h:h + 1].cpu(),
                                        v[:, h:h + 1].cpu(), scale)
        assert_bf16_attention(o[:, h:h + 1, rt], lse[:, h:h + 1, rt], o_ref, l_ref,
                              "video head %d" % h)
