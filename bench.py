"""Benchmark of the diffusion-transformer attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole hot path over the FLUX.1-dev 1024x1024
attention shape (B=1, H=24, N=4608 = 512 text + 4096 image tokens, D=128):
  1. attn_fwd, bf16, over the full K/V                       (O, LSE)
  2. the ring-step emulation: attn_fwd over 8 seeded uneven contiguous K/V
     chunks, then attn_merge of the 8 partials
  3. the fp8 variant: per-tensor quantisation of Q, K and V (one
     fp8_quant_per_tensor_multi call, two launches), then attn_fwd_fp8
  4. residual_diff over two bf16 [1, 4608, 3072] first-block residuals.
``value`` is the algorithmic attention work of the step (3 passes of
4*B*H*N*N*D FLOP) divided by the step's wall time with every input already
resident in HBM; the merge, quantisation and residual-diff kernels are
inside the timed region. ``roofline`` reports the dominant kernel (bf16
attn_fwd at the FLUX shape) from HIP events around each of its launches.
The 119056-token HunyuanVideo shape is timed separately (``video``: bf16 and
per-tensor fp8 attention).
``cpu_baseline`` times the float64 CPU oracle on a bounded sample.

Prints ONE JSON line.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s & % MFMA peak at 4608-tok FLUX and 119k-tok video shapes"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_flux_1024_traffic.json")
KERNEL_SOURCES = ["diffusion_transformer_attention_flash_amd/csrc/attn_fwd.hip",
                  "diffusion_transformer_attention_flash_amd/csrc/common.h"]


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    runs, or None when the kernel source has changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def attn_flop(B, H, Nq, Nkv, D):
    return 4.0 * B * H * Nq * Nkv * D


def cpu_baseline(q, k, v, scale, budget_s=12.0):
    """Time the float64 oracle on whole heads of the FLUX shape, as many heads
    as fit in about ``budget_s`` seconds (at least one)."""
    import numpy as np
    import oracle
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    B, H, N, D = q.shape
    done, t0 = 0, time.perf_counter()
    while done < H:
        oracle.attention(qc[:, done:done + 1], kc[:, done:done + 1], vc[:, done:done + 1], scale)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    return {
        "value": attn_flop(B, done, N, N, D) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads or cores,
        "kind": "oracle",
        "sample": "float64 numpy oracle.attention on %d of %d heads of the FLUX 4608-token "
                  "shape (all %d query rows each), %.1f s" % (done, H, N, dt),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--video-reps", type=int, default=3)
    ap.add_argument("--no-video", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", default="all",
                    help="comma-separated subset of attn,chunks,merge,quant,fp8,residual "
                         "(profiling runs only; the reported value needs all)")
    args = ap.parse_args()
    legs_on = set(["attn", "chunks", "merge", "quant", "fp8", "residual"]
                  if args.legs == "all" else args.legs.split(","))
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the ring/Ulysses exchanges are out of scope); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import diffusion_transformer_attention_flash_amd as dta
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    c2 = workloads.CONFIGS["flux_1024"]
    c3 = workloads.CONFIGS["flux_1024_chunked"]
    c5 = workloads.CONFIGS["flux_1024_fp8"]
    B, H, N, D = c2["B"], c2["H"], c2["N"], c2["D"]
    scale = D ** -0.5
    q, k, v = workloads.workload_qkv("flux_1024", device=dev)
    lens = workloads.chunk_lengths(c3["config"], N, c3["n_chunks"], c3["min_chunk"])
    chunks = workloads.split_kv(k, v, lens)
    n_parts = len(lens)
    o_parts = torch.empty((n_parts, B, H, N, D), dtype=torch.bfloat16, device=dev)
    l_parts = torch.empty((n_parts, B, H, N), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    o_m = torch.empty_like(q)
    l_m = torch.empty_like(lse)
    q8 = torch.empty(q.shape, dtype=torch.uint8, device=dev)
    k8 = torch.empty_like(q8)
    v8 = torch.empty_like(q8)
    ds = torch.empty(3, dtype=torch.float32, device=dev)
    o8 = torch.empty_like(q)
    l8 = torch.empty_like(lse)
    ra, rb = workloads.residual_pair(c5["config"], c5["residual_shape"], c5["residual_noise"], device=dev)
    rd = torch.empty((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    flop_full = attn_flop(B, H, N, N, D)
    step_flop = flop_full * sum(1 for x in ("attn", "chunks", "fp8") if x in legs_on)
    if "fp8" in legs_on and "quant" not in legs_on:
        for x, x8_, i in ((q, q8, 0), (k, k8, 1), (v, v8, 2)):
            dta.fp8_quant_per_tensor(x, x8_, ds[i:i + 1])

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if "attn" in legs_on:
            dta.attn_fwd(q, k, v, scale, o=o, lse=lse)
        if ev is not None:
            ev[1].record()
        if "chunks" in legs_on:
            for i, (kc, vc) in enumerate(chunks):
                dta.attn_fwd(q, kc, vc, scale, o=o_parts[i], lse=l_parts[i])
        if ev is not None:
            ev[2].record()
        if "merge" in legs_on:
            dta.attn_merge(o_parts, l_parts, o=o_m, lse=l_m)
        if ev is not None:
            ev[3].record()
        if "quant" in legs_on:
            dta.fp8_quant_per_tensor_multi([q, k, v], [q8, k8, v8], ds)
        if ev is not None:
            ev[4].record()
        if "fp8" in legs_on:
            dta.attn_fwd_fp8(q8, k8, v8, ds, scale, o=o8, lse=l8)
        if ev is not None:
            ev[5].record()
        if "residual" in legs_on:
            dta.residual_diff(ra, rb, out=rd)
        if ev is not None:
            ev[6].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K whole steps, bracketed by synchronisation.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # Per-leg HIP event timing over a second pass of K steps (same stream).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()

    def leg(a, b):
        return max(sum(e[a].elapsed_time(e[b]) for e in evs) / len(evs), 1e-6)

    ms_attn = leg(0, 1)
    ms_chunks = leg(1, 2)
    ms_merge = leg(2, 3)
    ms_quant = leg(3, 4)
    ms_fp8 = leg(4, 5)
    ms_res = leg(5, 6)
    merge_bytes = n_parts * (B * H * N * D * 2 + B * H * N * 4) + B * H * N * D * 2 + B * H * N * 4
    res_bytes = 2 * ra.numel() * 2
    quant_bytes = 3 * (2 * q.numel() * 2 + q.numel())     # amax read + cast read + fp8 write
    achieved = flop_full / (ms_attn * 1e-3) / 1e12
    traffic = load_traffic()

    legs = {
        "attn_fwd_bf16": {"ms": ms_attn, "TFLOP/s": achieved,
                          "frac_bf16_peak": achieved / PEAK_BF16_TFLOPS},
        "attn_fwd_bf16_8_chunks": {"ms": ms_chunks, "chunk_lens": lens,
                                   "TFLOP/s": flop_full / (ms_chunks * 1e-3) / 1e12},
        "attn_merge": {"ms": ms_merge, "GB/s": merge_bytes / (ms_merge * 1e-3) / 1e9,
                       "frac_hbm_peak": merge_bytes / (ms_merge * 1e-3) / 1e9 / PEAK_HBM_GBS,
                       "bytes": merge_bytes, "cache": "warm"},
        "fp8_quant_x3": {"ms": ms_quant, "GB/s": quant_bytes / (ms_quant * 1e-3) / 1e9,
                         "bytes": quant_bytes, "cache": "warm"},
        "attn_fwd_fp8": {"ms": ms_fp8, "TFLOP/s": flop_full / (ms_fp8 * 1e-3) / 1e12,
                         "frac_fp8_peak": flop_full / (ms_fp8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS},
        "residual_diff": {"ms": ms_res, "GB/s": res_bytes / (ms_res * 1e-3) / 1e9,
                          "frac_hbm_peak": res_bytes / (ms_res * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "bytes": res_bytes, "cache": "warm"},
    }

    leg_key = {"attn": "attn_fwd_bf16", "chunks": "attn_fwd_bf16_8_chunks",
               "merge": "attn_merge", "quant": "fp8_quant_x3", "fp8": "attn_fwd_fp8",
               "residual": "residual_diff"}
    legs = {leg_key[x]: legs[leg_key[x]] for x in leg_key if x in legs_on}

    # The HBM-bound kernels once more, each alone and cold: a 512 MB read
    # between repetitions evicts the 256 MB MALL (a read, so that no dirty
    # lines are left to write back during the timed kernel). A device copy of
    # the same byte count gives the bandwidth reachable at these sizes.
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    fsum = torch.empty((1,), dtype=torch.float32, device=dev)

    def cold_us(fn, reps=20):
        ts = []
        for r in range(reps + 2):
            torch.sum(flush, dim=(0,), out=fsum[0])
            a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_ev.record()
            fn()
            b_ev.record()
            torch.cuda.synchronize()
            if r >= 2:
                ts.append(a_ev.elapsed_time(b_ev) * 1e3)
        ts.sort()
        return ts[len(ts) // 2], ts[0]

    cold = {}
    if "merge" in legs_on:
        cold["attn_merge"] = (lambda: dta.attn_merge(o_parts, l_parts, o=o_m, lse=l_m), merge_bytes)
    if "quant" in legs_on:
        cold["fp8_quant_q"] = (lambda: dta.fp8_quant_per_tensor(q, q8, ds[0:1]), quant_bytes // 3)
    if "residual" in legs_on:
        cold["residual_diff"] = (lambda: dta.residual_diff(ra, rb, out=rd), res_bytes)
    if cold:
        cp_dst = torch.empty_like(ra)
        cold["device_copy_same_bytes_as_residual"] = (lambda: cp_dst.copy_(ra), res_bytes)
        for name, (fn, nbytes) in cold.items():
            med, mn = cold_us(fn)
            legs.setdefault("cold", {})[name] = {
                "us_median": med, "us_min": mn, "bytes": nbytes,
                "GB/s_median": nbytes / (med * 1e-6) / 1e9,
                "frac_hbm_peak": nbytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBS}
        del cp_dst
    del flush

    # First Block Cache step on the device (residual_diff + decision + the
    # guarded hidden += cached) at the FLUX residual shape, once with a
    # threshold that reuses the cache and once with one that does not.
    if "residual" in legs_on:
        hid = torch.zeros_like(ra)
        cac = torch.full_like(ra, 2.0 ** -9)
        fd = torch.empty((), dtype=torch.float32, device=dev)
        fu = torch.empty((), dtype=torch.int32, device=dev)
        fb = {}
        for label, thr in (("reuse", 1.0), ("recompute", 0.0)):
            fn = (lambda t: (lambda: dta.fbcache_step(ra, rb, t, hid, cac, diff=fd, use_cache=fu)))(thr)
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / args.steps * 1e3
            nbytes = res_bytes + (3 * ra.numel() * 2 if label == "reuse" else 0)
            fb[label] = {"us": us, "use_cache": int(fu.item()), "bytes": nbytes,
                         "GB/s": nbytes / (us * 1e-6) / 1e9}
        fb["in_step"] = False
        legs["fbcache_step"] = fb
        del hid, cac

    # Row-wise fp8 at the FLUX shape, outside the step: per-token power-of-two
    # Q/K scales applied by the MFMA operand scales with per-tensor V
    # (attn_fwd_fp8_rows), and with per-token V scales folded into per-block
    # scaled P (attn_fwd_fp8_rows_v).
    if "fp8" in legs_on:
        rq8 = torch.empty_like(q8)
        rk8 = torch.empty_like(q8)
        rv8 = torch.empty_like(q8)
        req = torch.empty((B, H, N), dtype=torch.uint8, device=dev)
        rek = torch.empty_like(req)
        rev = torch.empty_like(req)
        ro = torch.empty_like(q)
        rl = torch.empty_like(lse)
        dta.fp8_quant_rows_pow2(v, x8=rv8, e8m0=rev)
        rows_legs = {}
        for name, fn in (
                ("quant_rows_q_and_k", lambda: (dta.fp8_quant_rows_pow2(q, x8=rq8, e8m0=req),
                                                dta.fp8_quant_rows_pow2(k, x8=rk8, e8m0=rek))),
                ("attn_fwd_fp8_rows_v", lambda: dta.attn_fwd_fp8_rows_v(rq8, rk8, rv8, req, rek, rev,
                                                                        scale, o=ro, lse=rl)),
                ("attn_fwd_fp8_rows", lambda: dta.attn_fwd_fp8_rows(rq8, rk8, v8, req, rek, ds[2:3],
                                                                    scale, o=ro, lse=rl))):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            rows_legs[name] = {"ms": ms}
        qb = 2 * (q.numel() * 2 + q.numel() + B * H * N)
        rows_legs["quant_rows_q_and_k"]["GB/s"] = qb / (rows_legs["quant_rows_q_and_k"]["ms"] * 1e-3) / 1e9
        for kname in ("attn_fwd_fp8_rows", "attn_fwd_fp8_rows_v"):
            tf = flop_full / (rows_legs[kname]["ms"] * 1e-3) / 1e12
            rows_legs[kname]["TFLOP/s"] = tf
            rows_legs[kname]["frac_fp8_peak"] = tf / PEAK_FP8_TFLOPS
        rows_legs["in_step"] = False
        legs["fp8_rows"] = rows_legs
        del rq8, rk8, rv8, req, rek, rev, ro, rl

    # Layout kernels of context parallelism at the FLUX tensor size (P = 8):
    # Ulysses' head split of Q for the all-to-all, and the token concat of 8
    # received parts. Each moves 28.3 MB in and 28.3 MB out.
    if "attn" in legs_on:
        lay = {}
        heads8 = [H // 8] * 8
        toks8 = [N // 8] * 8
        buf_h = torch.empty(q.numel(), dtype=torch.bfloat16, device=dev)
        out_s = torch.empty_like(q)
        for name, fn in (("head_split_P8", lambda: dta.head_split(q, heads8, parts=buf_h)),
                         ("seq_concat_P8", lambda: dta.seq_concat(buf_h, toks8, B, H, D, out=out_s))):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / args.steps * 1e3
            nbytes = 2 * q.numel() * 2
            lay[name] = {"us": us, "bytes": nbytes, "GB/s": nbytes / (us * 1e-6) / 1e9,
                         "frac_hbm_peak": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
        lay["in_step"] = False
        legs["layout"] = lay
        del buf_h, out_s

    # The same ring with the merge fused into each step (attn_fwd_accum): the
    # first chunk by attn_fwd, the other seven folded into one running (o, lse).
    # Timed apart from the step, which keeps the separate partials + merge.
    if "chunks" in legs_on:
        o_r = torch.empty_like(q)
        l_r = torch.empty_like(lse)

        def ring():
            dta.attn_fwd(q, chunks[0][0], chunks[0][1], scale, o=o_r, lse=l_r)
            for kc, vc in chunks[1:]:
                dta.attn_fwd_accum(q, kc, vc, o_r, l_r, scale)

        for _ in range(3):
            ring()
        torch.cuda.synchronize()
        ra_ev, rb_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ra_ev.record()
        for _ in range(args.steps):
            ring()
        rb_ev.record()
        torch.cuda.synchronize()
        ms_ring = ra_ev.elapsed_time(rb_ev) / args.steps
        legs["ring_fused_8_steps"] = {
            "ms": ms_ring, "TFLOP/s": flop_full / (ms_ring * 1e-3) / 1e12,
            "vs_chunks_plus_merge_ms": ms_chunks + ms_merge,
            "in_step": False}
        del o_r, l_r
    video = None
    if not args.no_video:
        del chunks
        cv = workloads.CONFIGS["hunyuan_720p_129f"]
        qv, kv, vv = workloads.workload_qkv("hunyuan_720p_129f", device=dev)
        ov = torch.empty_like(qv)
        lv = torch.empty((cv["B"], cv["H"], cv["N"]), dtype=torch.float32, device=dev)
        dta.attn_fwd(qv, kv, vv, cv["D"] ** -0.5, o=ov, lse=lv)
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(1, args.video_reps)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dta.attn_fwd(qv, kv, vv, cv["D"] ** -0.5, o=ov, lse=lv)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ms_v = sorted(ts)[len(ts) // 2]
        fv = attn_flop(cv["B"], cv["H"], cv["N"], cv["N"], cv["D"])
        video = {"workload": "hunyuan_720p_129f (B=1, H=24, N=119056, D=128, bf16)",
                 "ms": ms_v, "TFLOP/s": fv / (ms_v * 1e-3) / 1e12,
                 "frac_bf16_peak": fv / (ms_v * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                 "reps": len(ts)}
        # The per-tensor fp8 attention at the same shape (quantisation outside
        # the timed launches).
        (q8v, k8v, v8v), dsv = dta.fp8_quant_per_tensor_multi([qv, kv, vv])
        del qv, kv, vv
        dta.attn_fwd_fp8(q8v, k8v, v8v, dsv, cv["D"] ** -0.5, o=ov, lse=lv)
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(1, args.video_reps)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dta.attn_fwd_fp8(q8v, k8v, v8v, dsv, cv["D"] ** -0.5, o=ov, lse=lv)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ms_v8 = sorted(ts)[len(ts) // 2]
        video["fp8_per_tensor"] = {"ms": ms_v8, "TFLOP/s": fv / (ms_v8 * 1e-3) / 1e12,
                                   "frac_fp8_peak": fv / (ms_v8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS}
        del q8v, k8v, v8v, ov, lv

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(q, k, v, scale)

    out = {
        "metric": METRIC,
        "value": step_flop / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "flux_1024: B=1, H=24, N=4608 (512 text + 4096 image tokens), D=128; "
                        "step = bf16 attention + 8-chunk ring-step emulation with merge + "
                        "fp8 (e4m3) quantise-and-attend + residual_diff on [1,4608,3072]",
            "global_batch": B,
            "seq_len": N,
            "heads": H,
            "head_dim": D,
            "step_attention_flop": step_flop,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "attn_fwd_bf16_kernel (flux_1024)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "legs": legs,
        "video": video,
        "wall_s_timed": wall,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
