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
