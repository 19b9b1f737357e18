"""The elementwise fp8 error bound of tests/helpers.py, pinned on the CPU.

The bound says how far an attention whose probabilities are rounded to E4M3
(at a fixed scale sigma against a reference max at most 2 bits below the row
max, or with one power-of-two scale per block of keys) may be from exact
attention on the same dequantised inputs. Here it must hold for the oracle's
own x448 rounding and for a CPU model of the kernels' x108 arithmetic with a
trailing reference max, and it must fail for plausible mistakes planted in
that model: too much slack in the reference max (108 p' saturates at 448),
V read one key off, and P rounded to 1 mantissa bit.
"""

import numpy as np
import pytest

import oracle
import workloads
from helpers import KERNEL_P_SCALE, fp8_p_rounding_bound


def _deq_inputs(q_gain, seed=3, n_q=64, n_kv=700, d=64):
    q, k, v = workloads.make_qkv(seed, 1, 2, n_q, n_kv, d, qknorm=True, q_gain=q_gain)
    (q8, sq), (k8, sk), (v8, sv) = (oracle.quant_per_tensor(t) for t in (q, k, v))
    qd = oracle.e4m3_decode(q8) * sq
    kd = oracle.e4m3_decode(k8) * sk
    vd = oracle.e4m3_decode(v8) * sv
    return (q8, k8, v8, (sq, sk, sv)), (qd, kd, vd)


def _model(qd, kd, vd, scale, sigma, lag_bits, rnd=oracle.e4m3_round, v_shift=0):
    """P rounded at x sigma against a reference max lag_bits (log2) below the
    row max; l from the unrounded p'. One head loop, float64."""
    B, H, nq, D = qd.shape
    o = np.empty((B, H, nq, D))
    for b in range(B):
        for h in range(H):
            s = scale * (qd[b, h] @ kd[b, h].T)
            m = s.max(axis=1, keepdims=True) - lag_bits * np.log(2.0)
            p = np.exp(s - m)
            vv = np.roll(vd[b, h], v_shift, axis=0)
            o[b, h] = (rnd(sigma * p) @ vv) / (sigma * p.sum(axis=1, keepdims=True))
    return o


@pytest.mark.parametrize("q_gain", [1.0, 4.0])
def test_oracle_x448_rounding_is_within_its_bound(q_gain):
    (q8, k8, v8, ds), (qd, kd, vd) = _deq_inputs(q_gain)
    scale = 64 ** -0.5
    o8, _ = oracle.attention_fp8(q8, k8, v8, ds, scale)
    o_star, bound = fp8_p_rounding_bound(qd, kd, vd, scale, p_scale=448.0)
    ratio = (np.abs(o8 - o_star) / bound).max()
    assert ratio <= 1.0
    assert ratio > 0.02                      # the bound is not vacuous here


@pytest.mark.parametrize("q_gain", [1.0, 4.0])
@pytest.mark.parametrize("lag", [0.0, 0.7, 2.0])
def test_kernel_arithmetic_model_is_within_the_bound(q_gain, lag):
    _, (qd, kd, vd) = _deq_inputs(q_gain)
    scale = 64 ** -0.5
    o = _model(qd, kd, vd, scale, KERNEL_P_SCALE, lag)
    o_star, bound = fp8_p_rounding_bound(qd, kd, vd, scale, p_scale=KERNEL_P_SCALE)
    assert (np.abs(o - o_star) <= bound).all()


def _round_1bit(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(np.abs(x))
    return np.sign(x) * np.ldexp(np.round(m * 4) / 4, e)


@pytest.mark.parametrize("mistake", ["saturating slack", "v one key off", "1-bit mantissa"])
def test_planted_mistakes_break_the_bound(mistake):
    _, (qd, kd, vd) = _deq_inputs(4.0)
    scale = 64 ** -0.5
    kw = {"saturating slack": dict(lag_bits=3.5),
          "v one key off": dict(lag_bits=1.0, v_shift=1),
          "1-bit mantissa": dict(lag_bits=1.0, rnd=_round_1bit)}[mistake]
    o = _model(qd, kd, vd, scale, KERNEL_P_SCALE, **kw)
    o_star, bound = fp8_p_rounding_bound(qd, kd, vd, scale, p_scale=KERNEL_P_SCALE)
    assert (np.abs(o - o_star) > bound).any()


def test_per_block_bound_holds_for_the_oracle_and_catches_a_wrong_block():
    """attention_fp8_rows_v at block 32 is within the block-32 bound, on
    random peaked inputs and on a constructed one; on the constructed one the
    same function at block 4096 (one scale per row) is not. There Q = 0
    (every p is 1), token 7 has a V scale 2^20 and is nonzero only in dims
    0..7, its 32-key block is otherwise all-zero V, and the other 480 tokens
    have V near 1 (scale 2^0): one scale per row flushes all of them (2^-20
    is beyond E4M3's span), blocks of 32 keep them."""
    import torch
    B, H, N, D = 1, 2, 256, 64
    q, k, v = workloads.make_qkv(9, B, H, N, N, D, q_gain=4.0)
    g = np.random.default_rng(2)
    v = v.float() * torch.from_numpy(np.exp2(g.integers(-12, 13, (B, H, N, 1))).astype(np.float32))

    def run(q, k, v, blocks):
        qr, eq = oracle.quant_rows_pow2(q, D)
        kr, ek = oracle.quant_rows_pow2(k, D)
        vr, ev = oracle.quant_rows_pow2(v, D)
        eq, ek, ev = eq.reshape(q.shape[:3]), ek.reshape(k.shape[:3]), ev.reshape(v.shape[:3])
        deq = lambda c, e: oracle.e4m3_decode(c) * np.exp2(e[..., None].astype(np.float64) - 127)
        o_star, bound = fp8_p_rounding_bound(deq(qr, eq), deq(kr, ek), deq(vr, ev), D ** -0.5,
                                             vq=oracle.e4m3_decode(vr),
                                             ev=ev.astype(np.int64) - 127, block=32)
        return [np.abs(oracle.attention_fp8_rows_v(qr, kr, vr, eq, ek, ev, D ** -0.5,
                                                   block=b)[0] - o_star) / bound
                for b in blocks]

    (r32,) = run(q, k, v, [32])
    assert r32.max() <= 1.0 and r32.max() > 0.02
    n = 512
    _, k2, _ = workloads.make_qkv(10, B, H, 1, n, D)
    q2 = torch.zeros(B, H, 64, D)
    v2 = 1.0 + 0.25 * torch.randn(B, H, n, D, generator=torch.Generator().manual_seed(6))
    v2[:, :, :32] = 0.0
    v2[:, :, 7, :8] = 2.0 ** 20
    r32, r_row = run(q2.to(torch.bfloat16), k2, v2.to(torch.bfloat16), [32, 4096])
    assert r32.max() <= 1.0
    assert r_row.max() > 5.0
