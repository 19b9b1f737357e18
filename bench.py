"""Benchmark of the diffusion-transformer attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--video-reps R]

Headline. ``value`` is the bf16 attention rate of ``attn_fwd`` at the
FLUX.1-dev 1024x1024 attention shape (B=1, H=24, N=4608 = 512 text + 4096
image tokens, D=128): 4*B*H*N*N*D FLOP divided by the median of that
launch's HIP-event durations over the K timed steps, with every input already
resident in HBM. ``video`` gives the same figure at the HunyuanVideo 720p x
129-frame shape (N = 119056 = 256 text + 33*45*80 video tokens), timed over
``--video-reps`` launches. Fractions are of MI355X's published dense bf16
MFMA peak (2.5 PFLOP/s); ``peaks`` adds the peak implied by the CU count and
the engine clock read on the box.

One step is one pass of the whole hot path over the FLUX shape:
  1. attn_fwd, bf16, over the full K/V                       (O, LSE)
  2. one ring's local work: attn_fwd over 8 seeded uneven contiguous K/V
     chunks, then attn_merge of the 8 partials
  3. the fp8 variant: per-tensor E4M3 quantisation of Q, K and V (one
     fp8_quant_per_tensor_multi call), then attn_fwd_fp8
  4. residual_diff over two bf16 [1, 4608, 3072] first-block residuals.
``ms_per_step`` is the whole step's time; every leg is timed with HIP events
on the launching stream inside the same timed steps (``legs``). The fp8
attention is reported against the fp8 peak only. The HBM-bound kernels are
also timed cold (a 512 MB read evicts the MALL between repetitions) beside
a cold read-only scan and a device copy of the same bytes (``cold``).
``roofline`` is the dominant kernel, bf16 attn_fwd at the FLUX shape, from
the mean of the same per-launch events. ``cpu_baseline`` times the float64
CPU oracle on bounded samples of the five configurations.

``shares`` times one GPU's share of the HunyuanVideo attention when it is
spread over 8 GPUs, at that share's real shape (no collective runs; the
exchanged buffers are built in place):
  * ulysses_8: 3 of the 24 heads over all 119 056 tokens. The received
    token shards are joined (seq_concat of Q, K and V), attn_fwd runs, and
    O is cut back into token shards (seq_split) for the return exchange.
  * ring_8: one rank's 14 882 query rows of all 24 heads against the 8 K/V
    shards in turn: attn_fwd on the first, attn_fwd_accum on the other 7.
Both do 1/8 of the video FLOPs.

Prints ONE JSON line.
"""

import argparse
import hashlib
import json
import math
import os
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s & % MFMA peak at 4608-tok FLUX and 119k-tok video shapes"
# MI355X published dense peaks (AMD specifications).
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0
# MFMA throughput per CU per engine clock on CDNA4 (dense).
BF16_FLOP_PER_CLK_CU = 4096
FP8_FLOP_PER_CLK_CU = 8192
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


def load_ceiling():
    """bench_ceiling.so (built by __graft_entry__.build()), or None."""
    import ctypes
    path = os.path.join(ROOT, "bench_ceiling.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.scan_read_only.restype = ctypes.c_int
    lib.scan_read_only.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return lib


def ctypes_ptr(addr):
    import ctypes
    return ctypes.c_void_p(addr)


def attn_flop(B, H, Nq, Nkv, D):
    return 4.0 * B * H * Nq * Nkv * D


def stats_ms(ts):
    ts = sorted(ts)
    return {"median_ms": statistics.median(ts), "min_ms": ts[0], "mean_ms": sum(ts) / len(ts),
            "max_ms": ts[-1], "reps": len(ts)}


# ---- engine clock and CU count, read on the box ---------------------------

def _run(cmd, timeout=20):
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout)
        return r.stdout
    except (OSError, subprocess.SubprocessError):
        return ""


def rocminfo_gpu():
    """(compute units, max engine clock in MHz) of the first gfx950 agent."""
    cus = mhz = None
    in_gpu = False
    for line in _run(["rocminfo"]).splitlines():
        s = line.strip()
        if s.startswith("Name:") and "gfx950" in s:
            in_gpu = True
        elif s.startswith("Agent ") and in_gpu and cus is not None:
            break
        if in_gpu and s.startswith("Compute Unit:") and cus is None:
            cus = int(s.split(":")[1])
        if in_gpu and s.startswith("Max Clock Freq. (MHz):") and mhz is None:
            mhz = int(s.split(":")[1])
    return cus, mhz


def current_sclk_mhz():
    """The engine clock the driver reports right now, in MHz, or None."""
    import glob
    import re
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            txt = open(f).read()
        except OSError:
            continue
        for line in txt.splitlines():
            if line.strip().endswith("*"):
                m = re.search(r"(\d+)\s*[Mm]hz", line)
                if m:
                    return int(m.group(1))
    return None


class ClockSampler:
    """Samples the reported engine clock from a host thread while the GPU
    runs a long stream of launches; the median is the clock under load."""

    def __init__(self, period_s=0.02):
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._loop, daemon=True)

    def _loop(self):
        while not self._stop.is_set():
            v = current_sclk_mhz()
            if v is not None:
                self.samples.append(v)
            time.sleep(self.period)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()

    def median(self):
        return statistics.median(self.samples) if self.samples else None


# ---- the CPU oracle baseline ----------------------------------------------

def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = threads = None
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                blas = "%s %s" % (p.get("internal_api"), p.get("version"))
                threads = p.get("num_threads")
                break
    except Exception:
        pass
    return {"cpu_model": model, "cores_available": len(os.sched_getaffinity(0)),
            "blas": blas, "blas_threads": threads}


def cpu_baseline(dev, scale):
    """The float64 oracle on bounded samples of the five configurations, on
    the host cores of this machine (BLAS-threaded). About 20-30 s in all."""
    import numpy as np
    import torch
    import oracle
    import workloads
    out = {}

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    # The tiny case (B=1, H=2, N=256, D=64), all rows, plus its 4-chunk merge.
    c = workloads.CONFIGS["tiny"]
    q, k, v = workloads.workload_qkv("tiny")
    sc = c["D"] ** -0.5

    def c1():
        oracle.attention(q, k, v, sc)
        parts = [oracle.attention(q, kc, vc, sc) for kc, vc in workloads.split_kv(k, v, c["chunks"])]
        oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    _, dt = timed(c1)
    out["tiny_256"] = {"s": dt, "sample": "all 2x256 rows, plus the 4x64-key chunked merge"}

    # FLUX 1024^2 bf16 (H=24, N=4608, D=128), whole heads, as many as fit in ~8 s.
    c = workloads.CONFIGS["flux_1024"]
    q, k, v = workloads.workload_qkv("flux_1024")
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    done, t0 = 0, time.perf_counter()
    while done < H:
        oracle.attention(q[:, done:done + 1], k[:, done:done + 1], v[:, done:done + 1], scale)
        done += 1
        if time.perf_counter() - t0 > 8.0:
            break
    dt = time.perf_counter() - t0
    flux_tflops = attn_flop(B, done, N, N, D) / dt / 1e12
    out["flux_1024"] = {"s": dt, "heads": done, "TFLOP/s": flux_tflops,
                           "sample": "%d of %d heads, all %d rows each" % (done, H, N)}

    # The FLUX K/V in 8 uneven chunks and their merge, head by head, as many heads
    # as fit in ~8 s.
    c3 = workloads.CONFIGS["flux_1024_chunked"]
    lens = workloads.chunk_lengths(c3["config"], N, c3["n_chunks"], c3["min_chunk"])
    done, t0 = 0, time.perf_counter()
    while done < H:
        hs = slice(done, done + 1)
        parts = [oracle.attention(q[:, hs], kc, vc, scale)
                 for kc, vc in workloads.split_kv(k[:, hs], v[:, hs], lens)]
        oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        done += 1
        if time.perf_counter() - t0 > 8.0:
            break
    dt = time.perf_counter() - t0
    out["flux_1024_8_chunks"] = {"s": dt, "heads": done,
                               "TFLOP/s": attn_flop(B, done, N, N, D) / dt / 1e12,
                               "sample": "%d of %d heads: 8 chunk attentions %s + merge"
                                         % (done, H, lens)}

    # The 119 056-token video shape, 256 rows per head (generated on the GPU as the
    # tests do, copied back head by head), for as many heads as fit in ~8 s.
    cv = workloads.CONFIGS["hunyuan_720p_129f"]
    qv, kv, vv = workloads.workload_qkv("hunyuan_720p_129f", device=dev)
    rows = workloads.sample_rows_per_head(cv["config"], cv["N"], cv["H"], cv["sample_rows"],
                                          cv["n_text"])
    done, busy, t0 = 0, 0.0, time.perf_counter()
    while done < cv["H"]:
        h = done
        rt = torch.from_numpy(rows[h]).to(dev)
        qh, kh, vh = qv[:, h:h + 1, rt].cpu(), kv[:, h:h + 1].cpu(), vv[:, h:h + 1].cpu()
        t1 = time.perf_counter()
        oracle.attention(qh, kh, vh, scale)
        busy += time.perf_counter() - t1
        done += 1
        if time.perf_counter() - t0 > 8.0:
            break
    del qv, kv, vv
    nv = cv["N"]
    flop_rows = attn_flop(1, done, rows.shape[1], nv, cv["D"])
    out["hunyuan_720p_129f"] = {"s": busy, "heads": done, "TFLOP/s": flop_rows / busy / 1e12,
                       "sample": "%d rows per head x %d of %d heads against all %d keys "
                                 "(oracle time only, not the host copies)"
                                 % (rows.shape[1], done, cv["H"], nv),
                       "extrapolated_full_tensor_s": busy * (nv / rows.shape[1]) * (cv["H"] / done),
                       "extrapolation": "x(119056/256 rows) x(24/heads): labelled estimate"}

    # The fp8 oracle on the FLUX tensors (per-tensor quantisation of the
    # whole Q, K and V, then attention head by head, as many heads as fit in
    # ~8 s), and the fp64 residual sum over the whole [1, 4608, 3072] pair.
    c5 = workloads.CONFIGS["flux_1024_fp8"]
    (qq, kk, vv8), dt_q = timed(lambda: [oracle.quant_per_tensor(t) for t in (q, k, v)])
    done, t0 = 0, time.perf_counter()
    while done < H:
        hs = slice(done, done + 1)
        oracle.attention_fp8(qq[0][:, hs], kk[0][:, hs], vv8[0][:, hs],
                             (qq[1], kk[1], vv8[1]), scale)
        done += 1
        if time.perf_counter() - t0 > 8.0:
            break
    dt = time.perf_counter() - t0
    ra, rb = workloads.residual_pair(c5["config"], c5["residual_shape"], c5["residual_noise"])
    (_, dt_r) = timed(lambda: oracle.residual_diff(ra, rb))
    res_bytes = 2 * ra.numel() * 2
    out["flux_1024_fp8_and_residual"] = {
        "quantise_s": dt_q, "fp8_attention_s": dt, "heads": done,
        "fp8_TFLOP/s": attn_flop(B, done, N, N, D) / dt / 1e12,
        "residual_s": dt_r, "residual_GB/s": res_bytes / dt_r / 1e9,
        "sample": "fp8 oracle: per-tensor quantisation of the whole Q, K, V, then attention on "
                  "%d of %d heads; residual_diff in fp64 over all %d elements"
                  % (done, H, ra.numel())}
    info = cpu_info()
    return {
        "value": flux_tflops,
        "unit": "TFLOP/s",
        "cores": info["blas_threads"] or info["cores_available"],
        "kind": "oracle",
        "sample": "float64 numpy oracle.attention on %s of the FLUX 4608-token shape; "
                  "the other configurations in 'configs'" % out["flux_1024"]["sample"],
        "configs": out,
        **info,
    }


def share_runs(qv, kv, vv, scale, reps, n_gpus=8):
    """One GPU's share of the attention on qv/kv/vv [1, H, N, D] spread over
    n_gpus GPUs, Ulysses (heads) and ring (query rows, K/V shards); see the
    module docstring. Returns timings in ms and rates."""
    import torch
    import diffusion_transformer_attention_flash_amd as dta
    B, H, N, D = qv.shape
    assert B == 1 and H % n_gpus == 0 and N % n_gpus == 0
    hs, n = H // n_gpus, N // n_gpus
    lens = [n] * n_gpus
    Ev = lambda: torch.cuda.Event(enable_timing=True)
    flop = attn_flop(1, H, N, N, D) / n_gpus

    def timed(fn, marks):
        fn()
        torch.cuda.synchronize()
        runs = []
        for _ in range(reps):
            ev = [Ev() for _ in range(marks + 1)]
            ev[0].record()
            fn(ev)
            runs.append(ev)
        torch.cuda.synchronize()
        return [[e[i].elapsed_time(e[i + 1]) for i in range(marks)] for e in runs]

    # Ulysses: the receive buffers of the all-to-all hold this GPU's heads of
    # every token shard, packed shard after shard.
    recv = [torch.cat([t[:, :hs, r * n:(r + 1) * n].reshape(-1) for r in range(n_gpus)])
            for t in (qv, kv, vv)]
    qkv = [torch.empty((1, hs, N, D), dtype=qv.dtype, device=qv.device) for _ in range(3)]
    o = torch.empty_like(qkv[0])
    lse = torch.empty((1, hs, N), dtype=torch.float32, device=qv.device)
    send = torch.empty(hs * N * D, dtype=qv.dtype, device=qv.device)

    def ulysses(ev=None):
        for src, dst in zip(recv, qkv):
            dta.seq_concat(src, lens, 1, hs, D, out=dst)
        if ev:
            ev[1].record()
        dta.attn_fwd(qkv[0], qkv[1], qkv[2], scale, o=o, lse=lse)
        if ev:
            ev[2].record()
        dta.seq_split(o, lens, parts=send)
        if ev:
            ev[3].record()

    t = timed(ulysses, 3)
    att = stats_ms([x[1] for x in t])
    uly = {"shape": "B=1, H=%d of %d, N=%d, D=%d" % (hs, H, N, D),
           "attn_fwd": {**att, "TFLOP/s_median": flop / (att["median_ms"] * 1e-3) / 1e12,
                        "frac_bf16_peak": flop / (att["median_ms"] * 1e-3) / 1e12
                        / PEAK_BF16_TFLOPS},
           "seq_concat_qkv_ms_median": statistics.median(x[0] for x in t),
           "seq_split_o_ms_median": statistics.median(x[2] for x in t),
           "total_ms_median": statistics.median(sum(x) for x in t),
           "layout_bytes": 2 * 4 * hs * N * D * 2}
    del recv, qkv, o, lse, send

    # Ring: rank 0's query rows; the K/V shards arrive in turn.
    qr = qv[:, :, :n].contiguous()
    ks = [kv[:, :, r * n:(r + 1) * n].contiguous() for r in range(n_gpus)]
    vs = [vv[:, :, r * n:(r + 1) * n].contiguous() for r in range(n_gpus)]
    o = torch.empty_like(qr)
    lse = torch.empty((1, H, n), dtype=torch.float32, device=qv.device)

    def ring(ev=None):
        dta.attn_fwd(qr, ks[0], vs[0], scale, o=o, lse=lse)
        if ev:
            ev[1].record()
        for r in range(1, n_gpus):
            dta.attn_fwd_accum(qr, ks[r], vs[r], o, lse, scale)
            if ev:
                ev[r + 1].record()

    t = timed(ring, n_gpus)
    tot = stats_ms([sum(x) for x in t])
    step_flop = flop / n_gpus
    rng = {"shape": "B=1, H=%d, Nq=%d per rank, %d K/V shards of %d, D=%d" % (H, n, n_gpus, n, D),
           **tot, "TFLOP/s_median": flop / (tot["median_ms"] * 1e-3) / 1e12,
           "frac_bf16_peak": flop / (tot["median_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "first_step_attn_fwd_ms_median": statistics.median(x[0] for x in t),
           "accum_step_ms_median": statistics.median(v for x in t for v in x[1:]),
           "step_TFLOP/s_median": step_flop / (statistics.median(v for x in t for v in x[1:])
                                               * 1e-3) / 1e12}
    del qr, ks, vs, o, lse
    return {"n_gpus": n_gpus, "flop_per_gpu": flop, "ulysses_8": uly, "ring_8": rng}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--video-reps", type=int, default=5)
    ap.add_argument("--no-video", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-shares", action="store_true",
                    help="skip the one-GPU shares of the 8-GPU video layouts "
                         "(built from the video tensors: --no-video skips them too)")
    ap.add_argument("--legs", default="all",
                    help="comma-separated subset of attn,chunks,merge,quant,fp8,residual "
                         "(profiling runs only; the step needs all)")
    args = ap.parse_args()
    legs_on = set(["attn", "chunks", "merge", "quant", "fp8", "residual"]
                  if args.legs == "all" else args.legs.split(","))
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the ring/Ulysses exchanges are out of scope); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("--steps must be >= 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import diffusion_transformer_attention_flash_amd as dta
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

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
    ra, rb = workloads.residual_pair(c5["config"], c5["residual_shape"], c5["residual_noise"],
                                     device=dev)
    rd = torch.empty((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    if "fp8" in legs_on and "quant" not in legs_on:
        dta.fp8_quant_per_tensor_multi([q, k, v], [q8, k8, v8], ds)

    flop_full = attn_flop(B, H, N, N, D)
    LEGS = ["attn", "chunks", "merge", "quant", "fp8", "residual"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        if "attn" in legs_on:
            dta.attn_fwd(q, k, v, scale, o=o, lse=lse)
        mark(1)
        if "chunks" in legs_on:
            for i, (kc, vc) in enumerate(chunks):
                dta.attn_fwd(q, kc, vc, scale, o=o_parts[i], lse=l_parts[i])
        mark(2)
        if "merge" in legs_on:
            dta.attn_merge(o_parts, l_parts, o=o_m, lse=l_m)
        mark(3)
        if "quant" in legs_on:
            dta.fp8_quant_per_tensor_multi([q, k, v], [q8, k8, v8], ds)
        mark(4)
        if "fp8" in legs_on:
            dta.attn_fwd_fp8(q8, k8, v8, ds, scale, o=o8, lse=l8)
        mark(5)
        if "residual" in legs_on:
            dta.residual_diff(ra, rb, out=rd)
        mark(6)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K whole steps bracketed by synchronisation. The per-leg
    # events are recorded on the launching stream inside the same steps.
    evs = [[Ev() for _ in range(7)] for _ in range(args.steps)]
    t_start, t_end = Ev(), Ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    per_leg = {name: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, name in enumerate(LEGS)}

    attn_st = stats_ms(per_leg["attn"])
    flux_tflops = flop_full / (attn_st["median_ms"] * 1e-3) / 1e12
    achieved = flop_full / (attn_st["mean_ms"] * 1e-3) / 1e12
    merge_bytes = n_parts * (B * H * N * D * 2 + B * H * N * 4) + B * H * N * D * 2 + B * H * N * 4
    res_bytes = 2 * ra.numel() * 2
    quant_bytes = 3 * (2 * q.numel() * 2 + q.numel())     # amax read + cast read + fp8 write

    def tf(flop, st):
        return {"TFLOP/s_median": flop / (st["median_ms"] * 1e-3) / 1e12,
                "TFLOP/s_best": flop / (st["min_ms"] * 1e-3) / 1e12}

    def gbs(nbytes, st):
        r = nbytes / (st["median_ms"] * 1e-3) / 1e9
        return {"GB/s_median": r, "frac_hbm_peak": r / PEAK_HBM_GBS, "bytes": nbytes,
                "cache": "warm (inside the step)"}

    legs = {}
    if "attn" in legs_on:
        legs["attn_fwd_bf16"] = {**attn_st, **tf(flop_full, attn_st),
                                 "frac_bf16_peak": flux_tflops / PEAK_BF16_TFLOPS}
    if "chunks" in legs_on:
        st = stats_ms(per_leg["chunks"])
        legs["attn_fwd_bf16_8_chunks"] = {**st, **tf(flop_full, st), "chunk_lens": lens,
                                          "frac_bf16_peak": flop_full / (st["median_ms"] * 1e-3)
                                          / 1e12 / PEAK_BF16_TFLOPS}
    if "merge" in legs_on:
        st = stats_ms(per_leg["merge"])
        legs["attn_merge"] = {**st, **gbs(merge_bytes, st)}
    if "quant" in legs_on:
        st = stats_ms(per_leg["quant"])
        legs["fp8_quant_qkv"] = {**st, **gbs(quant_bytes, st)}
    if "fp8" in legs_on:
        st = stats_ms(per_leg["fp8"])
        t8 = flop_full / (st["median_ms"] * 1e-3) / 1e12
        legs["attn_fwd_fp8"] = {**st, **tf(flop_full, st), "frac_fp8_peak": t8 / PEAK_FP8_TFLOPS,
                                "note": "e4m3 MFMA: against the fp8 peak, never the bf16 one"}
    if "residual" in legs_on:
        st = stats_ms(per_leg["residual"])
        legs["residual_diff"] = {**st, **gbs(res_bytes, st)}

    # The HBM-bound kernels once more, each alone and cold: a 512 MB read
    # between repetitions evicts the 256 MB MALL (a read, so no dirty lines
    # are written back during the timed kernel). Beside them, the ceilings a
    # kernel of the same size can reach: a read-only scan (torch's sum over
    # the same bytes) and a device copy.
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    fsum = torch.empty((1,), dtype=torch.float32, device=dev)

    def cold_us(fn, reps=20):
        ts = []
        for r in range(reps + 2):
            torch.sum(flush, dim=(0,), out=fsum[0])
            a_ev, b_ev = Ev(), Ev()
            a_ev.record()
            fn()
            b_ev.record()
            torch.cuda.synchronize()
            if r >= 2:
                ts.append(a_ev.elapsed_time(b_ev) * 1e3)
        ts.sort()
        return ts[len(ts) // 2], ts[0]

    cold = {}
    scan_src = torch.cat([ra.view(-1), rb.view(-1)])
    scan_out = torch.empty((), dtype=torch.float32, device=dev)
    cp_dst = torch.empty_like(ra)
    ceiling = load_ceiling()
    tag = torch.empty(8192, dtype=torch.int32, device=dev)
    cases = {}
    if "merge" in legs_on:
        cases["attn_merge"] = (lambda: dta.attn_merge(o_parts, l_parts, o=o_m, lse=l_m), merge_bytes)
    if "quant" in legs_on:
        cases["fp8_quant_q"] = (lambda: dta.fp8_quant_per_tensor(q, q8, ds[0:1]), quant_bytes // 3)
    if "residual" in legs_on:
        cases["residual_diff"] = (lambda: dta.residual_diff(ra, rb, out=rd), res_bytes)
        cases["torch_sum_same_bytes"] = (
            lambda: torch.sum(scan_src, dim=(0,), dtype=torch.float32, out=scan_out), res_bytes)
        cases["ceiling_device_copy_same_bytes"] = (lambda: cp_dst.copy_(ra), res_bytes)
    for name, (fn, nbytes) in cases.items():
        med, mn = cold_us(fn)
        cold[name] = {"us_median": med, "us_min": mn, "bytes": nbytes,
                      "GB/s_median": nbytes / (med * 1e-6) / 1e9,
                      "frac_hbm_peak": nbytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBS}
    if "residual" in legs_on and ceiling is not None:
        # The read-only ceiling: the fastest of a sweep of plain read-only
        # scans over the same 56.6 MB (grid x loads in flight per thread).
        sweep = {}
        stream = torch.cuda.current_stream(dev).cuda_stream
        for grid in (512, 1024, 2048, 4096):
            for unroll in (2, 4, 8):
                fn = (lambda g, u: lambda: ceiling.scan_read_only(
                    ctypes_ptr(scan_src.data_ptr()), res_bytes, ctypes_ptr(tag.data_ptr()),
                    g, u, ctypes_ptr(stream)))(grid, unroll)
                sweep["%dx%d" % (grid, unroll)] = cold_us(fn)[0]
        best = min(sweep, key=sweep.get)
        med = sweep[best]
        cold["ceiling_read_only_scan_same_bytes"] = {
            "us_median": med, "bytes": res_bytes, "config": "grid x unroll " + best,
            "GB/s_median": res_bytes / (med * 1e-6) / 1e9,
            "frac_hbm_peak": res_bytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "sweep_us_median": sweep}
        cold["residual_diff"]["frac_of_read_only_ceiling"] = med / cold["residual_diff"]["us_median"]
    del flush, scan_src, cp_dst, tag

    # The fused 8-step ring (attn_fwd_accum), apart from the step.
    ring = None
    if "chunks" in legs_on:
        o_r = torch.empty_like(q)
        l_r = torch.empty_like(lse)

        def ring_fn():
            dta.attn_fwd(q, chunks[0][0], chunks[0][1], scale, o=o_r, lse=l_r)
            for kc, vc in chunks[1:]:
                dta.attn_fwd_accum(q, kc, vc, o_r, l_r, scale)

        for _ in range(3):
            ring_fn()
        ts = []
        for _ in range(args.steps):
            a_ev, b_ev = Ev(), Ev()
            a_ev.record()
            ring_fn()
            b_ev.record()
            ts.append((a_ev, b_ev))
        torch.cuda.synchronize()
        st = stats_ms([a.elapsed_time(b) for a, b in ts])
        ring = {**st, **tf(flop_full, st)}
        del o_r, l_r
    del chunks

    # The HunyuanVideo shape: bf16 and per-tensor fp8, >= 5 launches each;
    # the engine clock is sampled while the bf16 launches run.
    cus, max_mhz = rocminfo_gpu()
    video = None
    shares = None
    load_mhz = None
    if not args.no_video:
        cv = workloads.CONFIGS["hunyuan_720p_129f"]
        qv, kv, vv = workloads.workload_qkv("hunyuan_720p_129f", device=dev)
        ov = torch.empty_like(qv)
        lv = torch.empty((cv["B"], cv["H"], cv["N"]), dtype=torch.float32, device=dev)
        sv = cv["D"] ** -0.5
        fv = attn_flop(cv["B"], cv["H"], cv["N"], cv["N"], cv["D"])
        dta.attn_fwd(qv, kv, vv, sv, o=ov, lse=lv)
        torch.cuda.synchronize()
        reps = max(5, args.video_reps)
        with ClockSampler() as clk:
            pairs = []
            for _ in range(reps):
                a_ev, b_ev = Ev(), Ev()
                a_ev.record()
                dta.attn_fwd(qv, kv, vv, sv, o=ov, lse=lv)
                b_ev.record()
                pairs.append((a_ev, b_ev))
            torch.cuda.synchronize()
        load_mhz = clk.median()
        st = stats_ms([a.elapsed_time(b) for a, b in pairs])
        video = {"workload": "hunyuan_720p_129f: B=1, H=24, N=119056 (256 text + 33x45x80 "
                             "video tokens), D=128, bf16 attn_fwd",
                 **st, **tf(fv, st),
                 "frac_bf16_peak": fv / (st["median_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        if not args.no_shares:
            del ov, lv
            shares = share_runs(qv, kv, vv, sv, reps)
            ov = torch.empty_like(qv)
            lv = torch.empty((cv["B"], cv["H"], cv["N"]), dtype=torch.float32, device=dev)
        (q8v, k8v, v8v), dsv = dta.fp8_quant_per_tensor_multi([qv, kv, vv])
        del qv, kv, vv
        dta.attn_fwd_fp8(q8v, k8v, v8v, dsv, sv, o=ov, lse=lv)
        torch.cuda.synchronize()
        pairs = []
        for _ in range(reps):
            a_ev, b_ev = Ev(), Ev()
            a_ev.record()
            dta.attn_fwd_fp8(q8v, k8v, v8v, dsv, sv, o=ov, lse=lv)
            b_ev.record()
            pairs.append((a_ev, b_ev))
        torch.cuda.synchronize()
        st = stats_ms([a.elapsed_time(b) for a, b in pairs])
        video["fp8_per_tensor"] = {**st, **tf(fv, st),
                                   "frac_fp8_peak": fv / (st["median_ms"] * 1e-3) / 1e12
                                   / PEAK_FP8_TFLOPS}
        del q8v, k8v, v8v, ov, lv

    n_cu = cus or torch.cuda.get_device_properties(dev).multi_processor_count
    peaks = {"published_bf16_TFLOP/s": PEAK_BF16_TFLOPS, "published_fp8_TFLOP/s": PEAK_FP8_TFLOPS,
             "compute_units": n_cu, "max_engine_clock_MHz": max_mhz,
             "engine_clock_under_load_MHz": load_mhz,
             "clock_source": "rocminfo (max); the driver's current engine-clock level sampled "
                             "while the video launches ran (under load)"}
    if max_mhz:
        peaks["bf16_TFLOP/s_at_max_clock"] = n_cu * max_mhz * 1e6 * BF16_FLOP_PER_CLK_CU / 1e12
    if load_mhz:
        p_load = n_cu * load_mhz * 1e6 * BF16_FLOP_PER_CLK_CU / 1e12
        peaks["bf16_TFLOP/s_at_load_clock"] = p_load
        peaks["flux_frac_of_load_clock_peak"] = flux_tflops / p_load
        if video:
            peaks["video_frac_of_load_clock_peak"] = video["TFLOP/s_median"] / p_load

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(dev, scale)

    traffic = load_traffic()
    out = {
        "metric": METRIC,
        "value": flux_tflops,
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
            "workload": "flux_1024: bf16 attn_fwd, B=1, H=24, N=4608 (512 text + 4096 image "
                        "tokens), D=128, QK-normalised N(0,1) Q/K, N(0,1) V; value = 4*B*H*N*N*D "
                        "FLOP / median launch time over the timed steps",
            "step": "bf16 attention + 8-chunk ring-step (8 attn_fwd + attn_merge) + per-tensor "
                    "fp8 quantise-and-attend + residual_diff on [1,4608,3072]",
            "global_batch": B,
            "seq_len": N,
            "heads": H,
            "head_dim": D,
            "parallelism": "single GPU",
        },
        "headline": {
            "flux_1024_bf16": {"TFLOP/s_median": flux_tflops,
                               "TFLOP/s_best": flop_full / (attn_st["min_ms"] * 1e-3) / 1e12,
                               "frac_bf16_peak": flux_tflops / PEAK_BF16_TFLOPS,
                               "median_ms": attn_st["median_ms"], "min_ms": attn_st["min_ms"],
                               "reps": attn_st["reps"]},
            "video_bf16": None if video is None else {
                "TFLOP/s_median": video["TFLOP/s_median"], "TFLOP/s_best": video["TFLOP/s_best"],
                "frac_bf16_peak": video["frac_bf16_peak"], "median_ms": video["median_ms"],
                "min_ms": video["min_ms"], "reps": video["reps"]},
        },
        "roofline": {
            "kernel": "attn_fwd_bf16_kernel (flux_1024)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "basis": "4*B*H*N*N*D FLOP per launch / mean HIP-event launch time over the timed steps",
        },
        "cpu_baseline": cpu,
        "peaks": peaks,
        "legs": legs,
        "cold": cold,
        "ring_fused_8_steps": ring,
        "video": video,
        "shares": shares,
        "wall_s_timed": wall,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
