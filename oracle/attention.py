"""Oracle: scaled-dot-product attention and the partial (O, LSE) merge, float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); never on the product
path.

Definitions (the pages name the operations but print no formula; the plain
textbook definition is taken, with natural-log LSE):

    s_ij = scale * sum_d q_id k_jd                  j = 0 .. Nkv-1
    O_i  = sum_j exp(s_ij) v_j / sum_j exp(s_ij)
    LSE_i = ln sum_j exp(s_ij)

* Attention: diffusers "Accelerate inference" guide, section "Scaled dot
  product attention" -- every SDPA backend computes this; non-causal, no
  mask and no dropout (the "Context parallelism" guide, section "Ring
  Anything Attention", requires attn_mask to be None and inference only).
* Merge: diffusers "Context parallelism" guide, section "Ring Attention" --
  each rank attends to the K/V block it holds, passes it on, and after a full
  turn has seen every token's K/V; the result must therefore equal attention
  over the concatenated K/V. With partials (O_p, LSE_p) over disjoint chunks,
  that exact identity is
      LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p.

Subtracting the row maximum before ``exp`` is the exact identity
exp(s - m)/sum exp(s - m) = exp(s)/sum exp(s); it only keeps float64 from
overflowing on peaked rows and is not a blocking or reordering of the sum.
"""

import numpy as np


def _as_f64(x):
    """Exact upcast to float64 (bf16/fp16/fp32 values are all representable)."""
    if hasattr(x, "detach"):  # a torch tensor: upcast in torch, then to numpy
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def softmax_rows(s):
    """Row softmax of logits ``s`` (last axis), plus the row max and row sum.

    Returns (p, m, l) with p = exp(s - m) / l, m = max_j s, l = sum_j exp(s - m).
    """
    s = np.asarray(s, dtype=np.float64)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    return e / l, m[..., 0], l[..., 0]


def attention(q, k, v, scale, rows=None):
    """Non-causal multi-head attention, O and natural-log LSE, in float64.

    q: [B, H, Nq, D]; k: [B, H, Nkv, D]; v: [B, H, Nkv, Dv] (any float dtype;
    upcast exactly; Dv = D in every workload).
    scale: the logit multiplier (1/sqrt(D) in every workload here).
    rows: optional 1-D array of query-row indices; only those rows are
          evaluated (query rows are independent), in the given order.

    Returns (O [B, H, len(rows) or Nq, Dv], LSE [B, H, len(rows) or Nq]).
    Nkv must be >= 1: attention over an empty key set is undefined.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or k.shape[:3] != v.shape[:3]:
        raise ValueError("q, k, v must be [B, H, N, D]; k and v share B, H, Nkv")
    B, H, Nq, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError("q and k/v disagree on B, H or D")
    if k.shape[2] < 1:
        raise ValueError("Nkv must be >= 1")
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        q = q[:, :, rows, :]
    nq = q.shape[2]
    o = np.empty((B, H, nq, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = float(scale) * (q[b, h] @ k[b, h].T)          # [nq, Nkv]
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            o[b, h] = (e @ v[b, h]) / l
            lse[b, h] = m[:, 0] + np.log(l[:, 0])
    return o, lse


def merge(o_parts, lse_parts):
    """Combine partial attention results over disjoint K/V chunks.

    o_parts: [n, B, H, Nq, D]; lse_parts: [n, B, H, Nq] (natural log).
    A partial whose LSE is -inf (attention over nothing) gets zero weight; a
    row whose partials are all -inf gets O = 0 and LSE = -inf.
    Returns (O [B, H, Nq, D], LSE [B, H, Nq]) in float64.
    """
    o_parts, lse_parts = _as_f64(o_parts), _as_f64(lse_parts)
    if o_parts.ndim != 5 or lse_parts.shape != o_parts.shape[:4]:
        raise ValueError("o_parts must be [n,B,H,Nq,D], lse_parts [n,B,H,Nq]")
    if o_parts.shape[0] < 1:
        raise ValueError("need at least one partial")
    big_m = lse_parts.max(axis=0)                              # [B, H, Nq]
    finite = np.isfinite(big_m)
    m_safe = np.where(finite, big_m, 0.0)
    with np.errstate(invalid="ignore"):
        w = np.where(np.isneginf(lse_parts), 0.0, np.exp(lse_parts - m_safe))
    wsum = w.sum(axis=0)                                       # [B, H, Nq]
    num = (w[..., None] * o_parts).sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(finite[..., None], num / np.where(finite, wsum, 1.0)[..., None], 0.0)
        lse = np.where(finite, m_safe + np.log(np.where(finite, wsum, 1.0)), -np.inf)
    return o, lse
