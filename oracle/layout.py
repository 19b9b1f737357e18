"""Oracle: the layout permutations of context parallelism, numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); never on the product
path.

Context parallelism guide, sections "Ulysses Attention", "Ulysses Anything
Attention" and "Ring Anything Attention": around the local attention each
rank splits its [B, H, N, D] tensor into per-rank parts along the heads or
the tokens, and concatenates the parts it receives along the other axis;
Ring Anything pads uneven token parts to a common length for the all-gather
and drops the padding afterwards. Parts are lists of numpy arrays here.
"""

import numpy as np


def _np(t):
    if hasattr(t, "detach"):
        return t.detach().to("cpu").numpy()
    return np.asarray(t)


def seq_concat(parts, lens):
    """Part p is [B, H, padded_p, D] with lens[p] valid tokens; the result is
    their valid tokens concatenated along axis 2, in part order."""
    return np.concatenate([_np(p)[:, :, :n] for p, n in zip(parts, lens)], axis=2)


def seq_split(x, lens, padded=None):
    """Inverse of seq_concat: part p holds tokens [sum(lens[:p]), +lens[p])
    followed by padded[p] - lens[p] rows of zeros."""
    x = _np(x)
    padded = list(lens) if padded is None else list(padded)
    out, start = [], 0
    for n, pad in zip(lens, padded):
        part = np.zeros(x.shape[:2] + (pad,) + x.shape[3:], dtype=x.dtype)
        part[:, :, :n] = x[:, :, start:start + n]
        out.append(part)
        start += n
    return out


def head_concat(parts):
    """Part p is [B, heads_p, N, D]; concatenated along axis 1."""
    return np.concatenate([_np(p) for p in parts], axis=1)


def head_split(x, heads):
    """Inverse of head_concat: part p holds heads [sum(heads[:p]), +heads[p])."""
    x = _np(x)
    cuts = np.cumsum(heads)[:-1]
    return np.split(x, cuts, axis=1)
