"""Oracle: First Block Cache residual difference, float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); never on the product
path.

ParaAttention guide, section "First Block Cache": the cache decision uses the
residual difference of the first transformer block's output between two
denoising steps as a proxy for how much the model output changes; when it is
small enough, the previous step's residual is reused. The relative measure
taken here is

    residual_diff(a, b) = mean|a - b| / mean|b| = sum|a - b| / sum|b|

over all elements (the element counts of the two means cancel), with ``a``
the current step's residual and ``b`` the previous one. sum|b| = 0 gives the
IEEE result (x/0 = +inf, 0/0 = NaN), so the host-side "diff < threshold"
comparison is false and the cache is not reused.
"""

import numpy as np


def residual_diff(a, b):
    """sum|a-b| / sum|b| in float64 over all elements of a and b."""
    if hasattr(a, "detach"):
        import torch
        a = a.detach().to("cpu").to(torch.float64).numpy()
        b = b.detach().to("cpu").to(torch.float64).numpy()
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    if a.shape != b.shape:
        raise ValueError("a and b must have the same number of elements")
    if a.size < 1:
        raise ValueError("need at least one element")
    num = np.abs(a - b).sum()
    den = np.abs(b).sum()
    with np.errstate(divide="ignore", invalid="ignore"):
        return float(np.float64(num) / np.float64(den))


def _bf16_round(x):
    """Round float64 values to the nearest bfloat16 (ties to even), returned as
    float64. bfloat16 keeps float32's 8-bit exponent and 7 stored mantissa
    bits; values beyond its largest finite value (about 3.39e38) become inf."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                    # x = m * 2**e, 0.5 <= |m| < 1
    # 8 significant bits: scale the mantissa to [128, 256), round half to even
    q = np.round(m * 256.0)               # numpy rounds halves to even
    out = np.ldexp(q / 256.0, e)
    # subnormal range of bf16 (below 2**-126): spacing is 2**-133
    tiny = np.abs(x) < 2.0 ** -126
    out = np.where(tiny, np.round(x * 2.0 ** 133) * 2.0 ** -133, out)
    with np.errstate(invalid="ignore"):
        out = np.where(np.abs(out) > 3.3895313892515355e38, np.sign(x) * np.inf, out)
    return np.where(np.isfinite(x), out, x)


def fbcache_step(r, r_prev, threshold, hidden, cached):
    """First Block Cache decision and cached-residual apply.

    ParaAttention guide, section "First Block Cache": the relative residual
    difference of the first block's output between this step (``r``) and the
    previous one (``r_prev``) decides whether the step reuses the cached
    residual of the remaining blocks; when it is small enough (below the
    threshold, 0.08 by default for FLUX) the remaining blocks are skipped and
    the cached residual is added to the first block's output ``hidden``.

    The decision is taken in float32, the precision of the device result:
    use = float32(diff) < float32(threshold); a NaN diff (sum|r_prev| = 0 and
    sum|r - r_prev| = 0) never reuses the cache. The update is one correctly
    rounded bfloat16 sum per element, hidden + cached.
    Returns (diff float64, use bool, new hidden float64 of bf16 values).
    """
    diff = residual_diff(r, r_prev)
    use = bool(np.float32(diff) < np.float32(threshold))
    h = np.asarray(hidden.detach().to("cpu").double().numpy() if hasattr(hidden, "detach")
                   else hidden, dtype=np.float64)
    c = np.asarray(cached.detach().to("cpu").double().numpy() if hasattr(cached, "detach")
                   else cached, dtype=np.float64)
    if h.shape != c.shape:
        raise ValueError("hidden and cached must have the same shape")
    out = _bf16_round(h + c) if use else h.copy()
    return diff, use, out
