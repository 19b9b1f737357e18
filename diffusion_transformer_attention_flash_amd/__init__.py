"""MI355X (gfx950) attention core of diffusion transformers.

Thin binding over libdta.so (include/dta.h): each function checks dtypes,
devices, shapes and contiguity, allocates outputs with torch if the caller
did not pass them, and hands raw device pointers plus the current HIP stream
to the C ABI. Every step of the computation runs in the library's HIP
kernels; there is no fallback path -- a missing library raises.

    attn_fwd(q, k, v, scale)              -> (o, lse)
    attn_merge(o_parts, lse_parts)        -> (o, lse)
    attn_fwd_accum(q, k, v, o, lse)       one ring step, merged into (o, lse)
    attn_merge_into(o, lse, o_part, lse_part)  pairwise in-place merge
    residual_diff(a, b)                   -> device float32 scalar
    residual_diff_noalloc(a, b, out)      the same, no workspace (library scratch)
    fbcache_step(r, r_prev, thr, hidden, cached) -> (diff, use_cache) on device
    seq_concat / seq_split / head_concat / head_split   layout permutations
    fp8_quant_per_tensor(x)               -> (x8 uint8, descale float32[1])
    fp8_quant_per_tensor_multi([q, k, v]) -> ([q8, k8, v8], descale float32[3])
    attn_fwd_fp8(q8, k8, v8, descale, scale) -> (o, lse)
    fp8_quant_rows_pow2(x)                -> (x8 uint8, e8m0 uint8 per row)
    attn_fwd_fp8_rows / attn_fwd_fp8_rows_v   row-wise scaled fp8 attention

The reductions share a small device workspace; the binding keeps one per
(device, stream), so calls on different streams never share it.
"""

import ctypes

import torch

from . import _lib
from ._lib import DtaError  # noqa: F401

__all__ = ["attn_fwd", "attn_merge", "attn_fwd_accum", "attn_merge_into", "residual_diff",
           "residual_diff_noalloc",
           "fbcache_step", "seq_concat", "seq_split", "head_concat", "head_split",
           "fp8_quant_rows_pow2", "attn_fwd_fp8_rows", "attn_fwd_fp8_rows_v",
           "fp8_quant_per_tensor", "fp8_quant_per_tensor_multi",
           "attn_fwd_fp8", "workspace", "DtaError"]

_workspaces = {}


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, name, dtype, ndim=None):
    """Type, dtype, rank and contiguity of one tensor argument (the device is
    checked once for all arguments by _gpu)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _out(t, name, dtype, shape):
    """A caller-supplied output (None: the binding allocates it): dtype,
    contiguity and the exact shape (a tuple) or element count (an int)."""
    if t is None:
        return
    _need(t, name, dtype)
    if isinstance(shape, int):
        if t.numel() != shape:
            raise ValueError("%s must hold %d elements, got shape %s" % (name, shape, tuple(t.shape)))
    elif tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _gpu(**named):
    """Every given tensor on one GPU (None entries are skipped)."""
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("%s must be on a GPU, got %s" % (name, t.device))
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s is on %s, the other tensors on %s" % (name, t.device, dev))


def _ptr(t):
    return ctypes_ptr(t.data_ptr())


def ctypes_ptr(addr):
    return ctypes.c_void_p(addr)


def workspace(device):
    """The reduction workspace of ``device`` for its current stream (allocated
    once per (device, stream) by torch). Kernels on one stream run in order,
    so they may share it; work on another stream gets its own."""
    device = torch.device(device)
    idx = device.index if device.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(idx).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None:
        nbytes = int(_lib.lib().dta_ws_bytes())
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=torch.device("cuda", idx))
        _workspaces[key] = ws
    return ws


def attn_fwd(q, k, v, scale=None, o=None, lse=None):
    """Non-causal attention: q [B,H,Nq,D], k/v [B,H,Nkv,D] bf16 -> (o bf16, lse f32)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    if tuple(k.shape) != (B, H, Nkv, D) or tuple(v.shape) != (B, H, Nkv, D):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    _out(o, "o", torch.bfloat16, (B, H, Nq, D))
    _out(lse, "lse", torch.float32, (B, H, Nq))
    _gpu(q=q, k=k, v=v, o=o, lse=lse)
    if scale is None:
        scale = D ** -0.5
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    st = _lib.lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                             B, H, Nq, Nkv, D, float(scale), ctypes_ptr(_stream(q)))
    _lib.check("attn_fwd", st)
    return o, lse


def attn_merge(o_parts, lse_parts, o=None, lse=None):
    """Combine packed partials o_parts [n,B,H,Nq,D] bf16, lse_parts [n,B,H,Nq] f32."""
    _need(o_parts, "o_parts", torch.bfloat16, 5)
    _need(lse_parts, "lse_parts", torch.float32, 4)
    n, B, H, Nq, D = o_parts.shape
    if tuple(lse_parts.shape) != (n, B, H, Nq):
        raise ValueError("lse_parts must be [n,B,H,Nq]")
    _out(o, "o", torch.bfloat16, (B, H, Nq, D))
    _out(lse, "lse", torch.float32, (B, H, Nq))
    _gpu(o_parts=o_parts, lse_parts=lse_parts, o=o, lse=lse)
    if o is None:
        o = torch.empty((B, H, Nq, D), dtype=torch.bfloat16, device=o_parts.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=o_parts.device)
    st = _lib.lib().attn_merge(_ptr(o_parts), _ptr(lse_parts), n, _ptr(o), _ptr(lse),
                               B, H, Nq, D, ctypes_ptr(_stream(o_parts)))
    _lib.check("attn_merge", st)
    return o, lse


def attn_fwd_accum(q, k, v, o, lse, scale=None):
    """One ring step fused: fold the attention of q over this k/v chunk into the
    running (o bf16 [B,H,Nq,D], lse f32 [B,H,Nq]) in place; returns (o, lse)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    if tuple(k.shape) != (B, H, Nkv, D) or tuple(v.shape) != (B, H, Nkv, D):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if o is None or lse is None:
        raise ValueError("attn_fwd_accum needs the running o and lse")
    _out(o, "o", torch.bfloat16, (B, H, Nq, D))
    _out(lse, "lse", torch.float32, (B, H, Nq))
    _gpu(q=q, k=k, v=v, o=o, lse=lse)
    if scale is None:
        scale = D ** -0.5
    st = _lib.lib().attn_fwd_accum(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   B, H, Nq, Nkv, D, float(scale), ctypes_ptr(_stream(q)))
    _lib.check("attn_fwd_accum", st)
    return o, lse


def attn_merge_into(o, lse, o_part, lse_part):
    """(o, lse) <- merge((o, lse), (o_part, lse_part)) in place; returns (o, lse)."""
    _need(o, "o", torch.bfloat16, 4)
    B, H, Nq, D = o.shape
    _out(lse, "lse", torch.float32, (B, H, Nq))
    _out(o_part, "o_part", torch.bfloat16, (B, H, Nq, D))
    _out(lse_part, "lse_part", torch.float32, (B, H, Nq))
    if lse is None or o_part is None or lse_part is None:
        raise ValueError("attn_merge_into needs o, lse, o_part and lse_part")
    _gpu(o=o, lse=lse, o_part=o_part, lse_part=lse_part)
    st = _lib.lib().attn_merge_into(_ptr(o), _ptr(lse), _ptr(o_part), _ptr(lse_part),
                                    B, H, Nq, D, ctypes_ptr(_stream(o)))
    _lib.check("attn_merge_into", st)
    return o, lse


def residual_diff(a, b, out=None):
    """sum|a-b| / sum|b| over all elements of bf16 a, b -> float32 device scalar."""
    _need(a, "a", torch.bfloat16)
    _need(b, "b", torch.bfloat16)
    if a.numel() != b.numel():
        raise ValueError("a and b must have the same number of elements")
    _out(out, "out", torch.float32, 1)
    _gpu(a=a, b=b, out=out)
    if out is None:
        out = torch.empty((), dtype=torch.float32, device=a.device)
    ws = workspace(a.device)
    st = _lib.lib().residual_diff(_ptr(a), _ptr(b), a.numel(), _ptr(out), _ptr(ws),
                                  ctypes_ptr(_stream(a)))
    _lib.check("residual_diff", st)
    return out


def residual_diff_noalloc(a, b, out):
    """residual_diff without a workspace: the library's own scratch array
    (for callers that cannot allocate; calls on one GPU must not overlap).
    ``out`` is a caller-allocated float32 device scalar."""
    _need(a, "a", torch.bfloat16)
    _need(b, "b", torch.bfloat16)
    if a.numel() != b.numel():
        raise ValueError("a and b must have the same number of elements")
    if out is None:
        raise ValueError("out is required (the call allocates nothing)")
    _out(out, "out", torch.float32, 1)
    _gpu(a=a, b=b, out=out)
    with torch.cuda.device(a.device):
        st = _lib.lib().residual_diff_noalloc(_ptr(a), _ptr(b), a.numel(), _ptr(out),
                                              ctypes_ptr(_stream(a)))
    _lib.check("residual_diff_noalloc", st)
    return out


def fbcache_step(r, r_prev, threshold, hidden, cached, diff=None, use_cache=None):
    """First Block Cache step on the device: diff = residual_diff(r, r_prev),
    use = diff < threshold, and hidden += cached (in place) when use.
    Returns (diff f32 scalar, use_cache int32 scalar), both device tensors."""
    _need(r, "r", torch.bfloat16)
    _need(r_prev, "r_prev", torch.bfloat16)
    _need(hidden, "hidden", torch.bfloat16)
    _need(cached, "cached", torch.bfloat16)
    if r.numel() != r_prev.numel():
        raise ValueError("r and r_prev must have the same number of elements")
    if hidden.numel() != cached.numel():
        raise ValueError("hidden and cached must have the same number of elements")
    _out(diff, "diff", torch.float32, 1)
    _out(use_cache, "use_cache", torch.int32, 1)
    _gpu(r=r, r_prev=r_prev, hidden=hidden, cached=cached, diff=diff, use_cache=use_cache)
    if diff is None:
        diff = torch.empty((), dtype=torch.float32, device=r.device)
    if use_cache is None:
        use_cache = torch.empty((), dtype=torch.int32, device=r.device)
    ws = workspace(r.device)
    st = _lib.lib().fbcache_step(_ptr(r), _ptr(r_prev), r.numel(), float(threshold),
                                 _ptr(hidden), _ptr(cached), hidden.numel(), _ptr(diff),
                                 _ptr(use_cache), _ptr(ws), ctypes_ptr(_stream(r)))
    _lib.check("fbcache_step", st)
    return diff, use_cache


def _host_ints(vals, name):
    vals = [int(x) for x in vals]
    if not vals:
        raise ValueError("%s must not be empty" % name)
    return (ctypes.c_int * len(vals))(*vals), len(vals)


def _layout_check(t, name, numel):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.element_size() != 2 or not t.is_contiguous():
        raise ValueError("%s must be a contiguous 16-bit tensor" % name)
    if t.numel() != numel:
        raise ValueError("%s has %d elements, expected %d" % (name, t.numel(), numel))


def seq_concat(parts, lens, B, H, D, padded=None, out=None):
    """Concatenate P token-parts (packed back to back, part p = [B,H,padded[p],D]
    with lens[p] valid tokens) into out [B,H,sum(lens),D]."""
    pads = list(lens) if padded is None else list(padded)
    _layout_check(parts, "parts", B * H * sum(pads) * D)
    if out is not None:
        _layout_check(out, "out", B * H * sum(lens) * D)
    _gpu(parts=parts, out=out)
    if out is None:
        out = torch.empty((B, H, sum(lens), D), dtype=parts.dtype, device=parts.device)
    cl, n = _host_ints(lens, "lens")
    cp, _ = _host_ints(pads, "padded")
    st = _lib.lib().seq_concat(_ptr(parts), _ptr(out), n, cl, cp, B, H, D,
                               ctypes_ptr(_stream(parts)))
    _lib.check("seq_concat", st)
    return out


def seq_split(x, lens, padded=None, parts=None):
    """Split x [B,H,sum(lens),D] along tokens into packed parts [B,H,padded[p],D]
    (padding rows zero); returns the flat packed buffer."""
    B, H, S, D = x.shape
    pads = list(lens) if padded is None else list(padded)
    _layout_check(x, "x", B * H * sum(lens) * D)
    if parts is not None:
        _layout_check(parts, "parts", B * H * sum(pads) * D)
    _gpu(x=x, parts=parts)
    if parts is None:
        parts = torch.empty(B * H * sum(pads) * D, dtype=x.dtype, device=x.device)
    cl, n = _host_ints(lens, "lens")
    cp, _ = _host_ints(pads, "padded")
    st = _lib.lib().seq_split(_ptr(x), _ptr(parts), n, cl, cp, B, H, D, ctypes_ptr(_stream(x)))
    _lib.check("seq_split", st)
    return parts


def head_concat(parts, heads, B, N, D, out=None):
    """Concatenate P head-parts (packed, part p = [B,heads[p],N,D]) into
    out [B,sum(heads),N,D]."""
    _layout_check(parts, "parts", B * sum(heads) * N * D)
    if out is not None:
        _layout_check(out, "out", B * sum(heads) * N * D)
    _gpu(parts=parts, out=out)
    if out is None:
        out = torch.empty((B, sum(heads), N, D), dtype=parts.dtype, device=parts.device)
    ch, n = _host_ints(heads, "heads")
    st = _lib.lib().head_concat(_ptr(parts), _ptr(out), n, ch, B, N, D, ctypes_ptr(_stream(parts)))
    _lib.check("head_concat", st)
    return out


def head_split(x, heads, parts=None):
    """Split x [B,sum(heads),N,D] along heads into packed parts [B,heads[p],N,D];
    returns the flat packed buffer."""
    B, Hs, N, D = x.shape
    _layout_check(x, "x", B * sum(heads) * N * D)
    if parts is not None:
        _layout_check(parts, "parts", x.numel())
    _gpu(x=x, parts=parts)
    if parts is None:
        parts = torch.empty(x.numel(), dtype=x.dtype, device=x.device)
    ch, n = _host_ints(heads, "heads")
    st = _lib.lib().head_split(_ptr(x), _ptr(parts), n, ch, B, N, D, ctypes_ptr(_stream(x)))
    _lib.check("head_split", st)
    return parts


def fp8_quant_per_tensor(x, x8=None, descale=None):
    """Per-tensor E4M3FN quantisation of bf16 x -> (x8 uint8 codes, descale f32[1])."""
    _need(x, "x", torch.bfloat16)
    _out(x8, "x8", torch.uint8, x.numel())
    _out(descale, "descale", torch.float32, 1)
    _gpu(x=x, x8=x8, descale=descale)
    if x8 is None:
        x8 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if descale is None:
        descale = torch.empty((1,), dtype=torch.float32, device=x.device)
    ws = workspace(x.device)
    st = _lib.lib().fp8_quant_per_tensor(_ptr(x), x.numel(), _ptr(x8), _ptr(descale),
                                         _ptr(ws), ctypes_ptr(_stream(x)))
    _lib.check("fp8_quant_per_tensor", st)
    return x8, descale


def fp8_quant_per_tensor_multi(xs, x8s=None, descale=None):
    """Per-tensor E4M3FN quantisation of up to four bf16 tensors (e.g. Q, K, V)
    in two launches -> (list of x8 uint8 codes, descale f32[len(xs)]); codes and
    scales equal fp8_quant_per_tensor's for each tensor."""
    xs = list(xs)
    if not 1 <= len(xs) <= 4:
        raise ValueError("fp8_quant_per_tensor_multi takes 1 to 4 tensors")
    for i, x in enumerate(xs):
        _need(x, "xs[%d]" % i, torch.bfloat16)
    if x8s is not None:
        x8s = list(x8s)
        if len(x8s) != len(xs):
            raise ValueError("x8s must match xs")
        for i, (x, x8) in enumerate(zip(xs, x8s)):
            _out(x8, "x8s[%d]" % i, torch.uint8, x.numel())
    _out(descale, "descale", torch.float32, len(xs))
    named = {"xs[%d]" % i: x for i, x in enumerate(xs)}
    named.update({"x8s[%d]" % i: t for i, t in enumerate(x8s or [])})
    _gpu(descale=descale, **named)
    dev = xs[0].device
    if x8s is None:
        x8s = [torch.empty(x.shape, dtype=torch.uint8, device=dev) for x in xs]
    if descale is None:
        descale = torch.empty((len(xs),), dtype=torch.float32, device=dev)
    n = len(xs)
    xp = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
    x8p = (ctypes.c_void_p * n)(*[t.data_ptr() for t in x8s])
    ns = (ctypes.c_int64 * n)(*[x.numel() for x in xs])
    ws = workspace(dev)
    st = _lib.lib().fp8_quant_per_tensor_multi(n, ctypes.cast(xp, ctypes.c_void_p),
                                               ctypes.cast(ns, ctypes.c_void_p),
                                               ctypes.cast(x8p, ctypes.c_void_p), _ptr(descale),
                                               _ptr(ws), ctypes_ptr(_stream(xs[0])))
    _lib.check("fp8_quant_per_tensor_multi", st)
    return x8s, descale


def _fp8_qkv(q8, k8, v8):
    _need(q8, "q8", torch.uint8, 4)
    _need(k8, "k8", torch.uint8, 4)
    _need(v8, "v8", torch.uint8, 4)
    B, H, Nq, D = q8.shape
    Nkv = k8.shape[2]
    if tuple(k8.shape) != (B, H, Nkv, D) or tuple(v8.shape) != (B, H, Nkv, D):
        raise ValueError("shape mismatch: q8 %s k8 %s v8 %s"
                         % (tuple(q8.shape), tuple(k8.shape), tuple(v8.shape)))
    return B, H, Nq, Nkv, D


def _attn_outputs(o, lse, B, H, Nq, D, device):
    if o is None:
        o = torch.empty((B, H, Nq, D), dtype=torch.bfloat16, device=device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=device)
    return o, lse


def attn_fwd_fp8(q8, k8, v8, descale, scale=None, o=None, lse=None):
    """fp8 attention: E4M3FN codes (uint8) q8/k8/v8, descale f32[3] = (s_q, s_k, s_v)."""
    B, H, Nq, Nkv, D = _fp8_qkv(q8, k8, v8)
    _out(descale, "descale", torch.float32, 3)
    if descale is None:
        raise ValueError("descale must hold 3 floats (s_q, s_k, s_v)")
    _out(o, "o", torch.bfloat16, (B, H, Nq, D))
    _out(lse, "lse", torch.float32, (B, H, Nq))
    _gpu(q8=q8, k8=k8, v8=v8, descale=descale, o=o, lse=lse)
    if scale is None:
        scale = D ** -0.5
    o, lse = _attn_outputs(o, lse, B, H, Nq, D, q8.device)
    st = _lib.lib().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(descale), _ptr(o),
                                 _ptr(lse), B, H, Nq, Nkv, D, float(scale),
                                 ctypes_ptr(_stream(q8)))
    _lib.check("attn_fwd_fp8", st)
    return o, lse


def fp8_quant_rows_pow2(x, row_len=None, x8=None, e8m0=None):
    """Row-wise E4M3 quantisation with power-of-two scales. Rows are the
    last dimension of x unless row_len is given. Returns (x8 uint8 with x's
    shape, e8m0 uint8 [rows]); the scale of row r is 2^(e8m0[r] - 127)."""
    _need(x, "x", torch.bfloat16)
    if row_len is None:
        row_len = x.shape[-1]
    if row_len < 1 or x.numel() % row_len:
        raise ValueError("row_len must divide the element count")
    rows = x.numel() // row_len
    _out(x8, "x8", torch.uint8, x.numel())
    _out(e8m0, "e8m0", torch.uint8, rows)
    _gpu(x=x, x8=x8, e8m0=e8m0)
    if x8 is None:
        x8 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if e8m0 is None:
        e8m0 = torch.empty(x.shape[:-1] if row_len == x.shape[-1] else (rows,),
                           dtype=torch.uint8, device=x.device)
    st = _lib.lib().fp8_quant_rows_pow2(_ptr(x), rows, int(row_len), _ptr(x8), _ptr(e8m0),
                                        ctypes_ptr(_stream(x)))
    _lib.check("fp8_quant_rows_pow2", st)
    return x8, e8m0


def attn_fwd_fp8_rows(q8, k8, v8, q_e8m0, k_e8m0, v_descale, scale=None, o=None, lse=None):
    """fp8 attention with per-token power-of-two Q/K scales (E8M0 bytes
    [B,H,N]) and V's per-tensor scale (f32[1])."""
    B, H, Nq, Nkv, D = _fp8_qkv(q8, k8, v8)
    for t, name, n in ((q_e8m0, "q_e8m0", B * H * Nq), (k_e8m0, "k_e8m0", B * H * Nkv)):
        if t is None:
            raise ValueError("%s is required" % name)
        _out(t, name, torch.uint8, n)
    if v_descale is None:
        raise ValueError("v_descale is required")
    _out(v_descale, "v_descale", torch.float32, 1)
    _out(o, "o", torch.bfloat16, (B, H, Nq, D))
    _out(lse, "lse", torch.float32, (B, H, Nq))
    _gpu(q8=q8, k8=k8, v8=v8, q_e8m0=q_e8m0, k_e8m0=k_e8m0, v_descale=v_descale, o=o, lse=lse)
    if scale is None:
        scale = D ** -0.5
    o, lse = _attn_outputs(o, lse, B, H, Nq, D, q8.device)
    st = _lib.lib().attn_fwd_fp8_rows(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_e8m0), _ptr(k_e8m0),
                                      _ptr(v_descale), _ptr(o), _ptr(lse), B, H, Nq, Nkv, D,
                                      float(scale), ctypes_ptr(_stream(q8)))
    _lib.check("attn_fwd_fp8_rows", st)
    return o, lse


def attn_fwd_fp8_rows_v(q8, k8, v8, q_e8m0, k_e8m0, v_e8m0, scale=None, o=None, lse=None):
    """fp8 attention with per-token power-of-two scales for Q, K and V (E8M0
    bytes [B,H,N]) and per-block power-of-two P scales."""
    B, H, Nq, Nkv, D = _fp8_qkv(q8, k8, v8)
    for t, name, n in ((q_e8m0, "q_e8m0", B * H * Nq), (k_e8m0, "k_e8m0", B * H * Nkv),
                       (v_e8m0, "v_e8m0", B * H * Nkv)):
        if t is None:
            raise ValueError("%s is required" % name)
        _out(t, name, torch.uint8, n)
    _out(o, "o", torch.bfloat16, (B, H, Nq, D))
    _out(lse, "lse", torch.float32, (B, H, Nq))
    _gpu(q8=q8, k8=k8, v8=v8, q_e8m0=q_e8m0, k_e8m0=k_e8m0, v_e8m0=v_e8m0, o=o, lse=lse)
    if scale is None:
        scale = D ** -0.5
    o, lse = _attn_outputs(o, lse, B, H, Nq, D, q8.device)
    st = _lib.lib().attn_fwd_fp8_rows_v(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_e8m0), _ptr(k_e8m0),
                                        _ptr(v_e8m0), _ptr(o), _ptr(lse), B, H, Nq, Nkv, D,
                                        float(scale), ctypes_ptr(_stream(q8)))
    _lib.check("attn_fwd_fp8_rows_v", st)
    return o, lse
