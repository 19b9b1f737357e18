"""Shared gates and comparison helpers for the parity tests.

Stated tolerances (the hot path's contract):
  bf16 attention: O max-abs error <= 2e-2, LSE abs error <= 1e-3, against the
                  float64 oracle on the exact bf16 inputs the kernel reads;
  fp8 attention:  O mean-abs error <= 5e-2;
  residual_diff:  relative error <= 1e-4.
Random-input O is small (|O| ~ sqrt(e/N)), so the stated O gates alone would
pass an all-zero output; the internal gates below add a relative-L2 bound and
run peaked inputs whose O is O(1).
"""

import numpy as np
import torch

O_MAX_ABS = 2e-2
LSE_ABS = 1e-3
FP8_O_MEAN_ABS = 5e-2
RESIDUAL_REL = 1e-4
# internal gates
O_REL_L2 = 1e-2
FP8_REL_L2_VS_BF16 = 0.10
FP8_REL_L2_VS_DEQUANT = 0.05
# Peaked rows (logit spread x4) amplify the E4M3 rounding of Q and K into the
# logits, so the total fp8 error against the bf16-input oracle doubles; the
# kernel-arithmetic gate against the dequantised oracle stays at 0.05.
FP8_REL_L2_VS_BF16_PEAKED = 0.20


def to64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def rel_l2(x, ref):
    x, ref = to64(x), to64(ref)
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def assert_bf16_attention(o, lse, o_ref, lse_ref, what=""):
    o, lse, o_ref, lse_ref = to64(o), to64(lse), to64(o_ref), to64(lse_ref)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), what + ": non-finite output"
    e_o = np.abs(o - o_ref).max()
    e_l = np.abs(lse - lse_ref).max()
    r = rel_l2(o, o_ref)
    msg = "%s: O max-abs %.3e, LSE max-abs %.3e, O rel-L2 %.3e" % (what, e_o, e_l, r)
    print(msg)
    assert e_o <= O_MAX_ABS, msg
    assert e_l <= LSE_ABS, msg
    assert r <= O_REL_L2, msg
    return e_o, e_l, r
