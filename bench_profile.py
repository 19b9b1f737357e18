"""Helpers for the rocprofv3 evidence behind bench.py's roofline figures.

    python bench_profile.py copy [--mib 1024] [--reps 5]
        A plain device-to-device copy of known size (reads and writes MIB
        MiB each per launch): the reference that scales the FETCH_SIZE and
        WRITE_SIZE counters to bytes.
    python bench_profile.py nkv-sweep [--nkv 1,64,...] [--reps 20]
        bf16 attn_fwd at the FLUX query shape over a list of K/V lengths
        (the fixed cost of a launch against its per-tile cost).
    python bench_profile.py summarize-sweep DIR OUT.md --cmd "..."
        Median duration per K/V length from that sweep's kernel trace and a
        least-squares line fixed + per-tile.
    python bench_profile.py balance-probe [--reps 20]
        bf16 attn_fwd at four shapes of one kernel, interleaved: the FLUX
        launch (432 workgroups, 72 K/V tiles each), its first round alone
        (256 workgroups), its second round alone (176 workgroups), and the
        same FLOPs spread evenly over 256 workgroups (121.5 tiles each), the
        bound of any split-K schedule of the FLUX launch.
    python bench_profile.py summarize-balance DIR OUT.md --cmd "..."
        Median duration per shape from that probe's kernel trace.
    python bench_profile.py summarize-trace DIR OUT.md --cmd "..."
        Turns a `rocprofv3 --kernel-trace --stats -f csv` directory into a
        short markdown table (launches, average, median and total time per
        kernel, grid and position in a run of back-to-back launches).
    python bench_profile.py summarize-pmc --fetch DIR --write DIR
            --copy-fetch DIR --copy-write DIR --kernel REGEX [--grid N]
            [--first-of-run] --out OUT.json --cmd "..."
        Per-launch HBM bytes of one kernel from FETCH_SIZE / WRITE_SIZE runs,
        each scaled by what the same counter reads for the copy above.
    python bench_profile.py summarize-counters --dir DIR [--dir DIR ...]
            --sel "LABEL|REGEX|GRID|PLACE" [--sel ...]
            --out OUT.md --title "..." --cmd "..."
        Median per dispatch of every counter found in the counter directories,
        for each selection of kernels (name regex, grid size or *, and the
        dispatch's place in a run of consecutive dispatches of one kernel:
        first, later or any, optionally :N for runs of length N).
"""

import argparse
import csv
import glob
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))


def cmd_copy(args):
    import torch
    n = args.mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 2, "copy_bytes_written": n * 2, "reps": args.reps}))


SWEEP_NKV = (1, 64, 128, 256, 576, 1152, 2304, 4608)


def _sweep_nkv(arg):
    return [int(x) for x in arg.split(",")] if arg else list(SWEEP_NKV)


def cmd_nkv_sweep(args):
    """bf16 attn_fwd at the FLUX query shape (B=1, H=24, Nq=4608, D=128)
    over a list of K/V lengths: for each, 3 warm-up launches then --reps
    launches, in order, with a synchronisation between lengths (the order
    summarize-sweep relies on)."""
    import torch
    sys.path.insert(0, ROOT)
    import diffusion_transformer_attention_flash_amd as dta
    import workloads
    dev = torch.device("cuda", 0)
    q, _, _ = workloads.make_qkv(2, 1, 24, 4608, 8, 128, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((1, 24, 4608), dtype=torch.float32, device=dev)
    for nkv in _sweep_nkv(args.nkv):
        _, k, v = workloads.make_qkv(2, 1, 24, 8, nkv, 128, device=dev)
        torch.cuda.synchronize()
        for _ in range(3 + args.reps):
            dta.attn_fwd(q, k, v, 128 ** -0.5, o=o, lse=lse)
        torch.cuda.synchronize()
    print(json.dumps({"nkv": _sweep_nkv(args.nkv), "reps": args.reps}))


BALANCE_SHAPES = (
    # (label, H, Nq, Nkv): B = 1, D = 128, 256 query rows per workgroup
    ("FLUX launch: 432 workgroups x 72 tiles", 24, 4608, 4608),
    ("first round alone: 256 x 72 tiles", 16, 4096, 4608),
    ("second round alone: 176 x 72 tiles", 11, 4096, 4608),
    ("equal FLOPs balanced: 256 x 121.5 tiles", 16, 4096, 7776),
)


def cmd_balance_probe(args):
    """The shapes of BALANCE_SHAPES, launched in turn --reps times after 3
    warm-up turns, so that clock drift falls on all of them alike."""
    import torch
    sys.path.insert(0, ROOT)
    import diffusion_transformer_attention_flash_amd as dta
    import workloads
    dev = torch.device("cuda", 0)
    cases = []
    for _, h, nq, nkv in BALANCE_SHAPES:
        q, _, _ = workloads.make_qkv(2, 1, h, nq, 8, 128, device=dev)
        _, k, v = workloads.make_qkv(2, 1, h, 8, nkv, 128, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty((1, h, nq), dtype=torch.float32, device=dev)
        cases.append((q, k, v, o, lse))
    torch.cuda.synchronize()
    for _ in range(3 + args.reps):
        for q, k, v, o, lse in cases:
            dta.attn_fwd(q, k, v, 128 ** -0.5, o=o, lse=lse)
    torch.cuda.synchronize()
    print(json.dumps({"shapes": [c[0] for c in BALANCE_SHAPES], "reps": args.reps}))


def cmd_summarize_balance(args):
    """Median attn_fwd duration per shape of the balance-probe's kernel trace
    (launches cycle through BALANCE_SHAPES in order)."""
    rows = []
    for path in _find(args.dir, "kernel_trace.csv"):
        with open(path) as f:
            rows += [r for r in csv.DictReader(f) if "attn_fwd_bf16_kernel" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    ns = len(BALANCE_SHAPES)
    if len(rows) != ns * (3 + args.reps):
        raise SystemExit("expected %d attn_fwd launches, found %d" % (ns * (3 + args.reps), len(rows)))
    timed = rows[3 * ns:]
    lines = ["# rocprofv3 kernel trace: %s" % args.title, "", args.cmd, "",
             "| shape (B=1, D=128) | H | Nq | Nkv | launches | median (us) | min (us) | TFLOP/s at median |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for i, (label, h, nq, nkv) in enumerate(BALANCE_SHAPES):
        d = sorted(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in timed[i::ns])
        med = d[len(d) // 2] / 1e3
        flops = 4.0 * h * nq * nkv * 128
        lines.append("| %s | %d | %d | %d | %d | %.2f | %.2f | %.1f |" % (
            label, h, nq, nkv, len(d), med, d[0] / 1e3, flops / med / 1e6))
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_summarize_sweep(args):
    """Median attn_fwd duration per K/V length from the nkv-sweep's kernel
    trace, and the least-squares line time = fixed + per_tile * tiles
    (tiles = ceil(Nkv / 64))."""
    rows = []
    for path in _find(args.dir, "kernel_trace.csv"):
        with open(path) as f:
            rows += [r for r in csv.DictReader(f) if "attn_fwd_bf16_kernel" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    nkvs = _sweep_nkv(args.nkv)
    per = 3 + args.reps
    if len(rows) != per * len(nkvs):
        raise SystemExit("expected %d attn_fwd launches, found %d" % (per * len(nkvs), len(rows)))
    lines = ["# rocprofv3 kernel trace: %s" % args.title, "",
             "Command (repo root): `%s`" % args.cmd, "",
             "| Nkv | 64-key tiles | launches | median (us) | min (us) |", "|---:|---:|---:|---:|---:|"]
    xs, ys = [], []
    for i, nkv in enumerate(nkvs):
        d = sorted(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                   for r in rows[i * per + 3:(i + 1) * per])
        med = d[len(d) // 2] / 1e3
        tiles = -(-nkv // 64)
        xs.append(tiles)
        ys.append(med)
        lines.append("| %d | %d | %d | %.2f | %.2f |" % (nkv, tiles, len(d), med, d[0] / 1e3))
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    slope = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
    fixed = my - slope * mx
    lines += ["", "Least-squares line over all lengths: %.2f us fixed + %.3f us per 64-key tile "
              "(432 workgroups of 256 query rows)." % (fixed, slope)]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit("no *%s under %s" % (suffix, d))
    return hits


def _col(row, *keys):
    for k in row:
        kl = k.lower().replace("_", "")
        if all(x in kl for x in keys):
            return k
    raise KeyError(keys)


def cmd_summarize_trace(args):
    """Per-kernel statistics from the kernel trace. Launches of one kernel
    that follow each other directly form a run; launches are grouped by run
    length and by whether they open the run (bench.py's step launches the
    full-K/V attention first, then the 8 chunk attentions with the same grid:
    a run of 9 whose first launch is the full attention)."""
    rows = []
    for path in _find(args.dir, "kernel_trace.csv"):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise SystemExit("empty trace")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    # Runs: maximal sequences of consecutive launches of one kernel. A launch
    # is labelled by its run's length and whether it opens the run.
    runs, cur = [], []
    for r in rows:
        if cur and r["Kernel_Name"] != cur[-1]["Kernel_Name"]:
            runs.append(cur)
            cur = []
        cur.append(r)
    if cur:
        runs.append(cur)
    groups = {}
    for run in runs:
        for pos, r in enumerate(run):
            grid = r.get("Grid_Size_X") or r.get("Grid_Size") or "?"
            where = ("first of run of %d" if pos == 0 else "later in run of %d") % len(run)
            key = (r["Kernel_Name"], grid, where)
            groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = ["# rocprofv3 kernel trace: %s" % args.title, "",
             "Command (repo root): `%s`" % args.cmd, "",
             "| kernel | grid (threads) | launches | calls | average (us) | median (us) | total (ms) |",
             "|---|---:|---|---:|---:|---:|---:|"]
    for (name, grid, where), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) <= 90 else name[:87] + "..."
        d_sorted = sorted(d)
        lines.append("| `%s` | %s | %s | %d | %.2f | %.2f | %.3f |" % (
            short, grid, where, len(d), statistics.mean(d) / 1e3,
            d_sorted[len(d) // 2] / 1e3, sum(d) / 1e6))
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _pmc_values(d, counter, kernel_re, grid=None, first_of_run=False):
    """Counter value per dispatch of kernels matching kernel_re (and grid).
    With first_of_run, only dispatches that start a run of consecutive
    dispatches of the same kernel count (see cmd_summarize_trace)."""
    rows = []
    for path in _find(d, "counter_collection.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get(_col(r, "counter", "name")) == counter:
                    rows.append(r)
    if not rows:
        raise SystemExit("no %s rows in %s" % (counter, d))
    did = _col(rows[0], "dispatch", "id")
    rows.sort(key=lambda r: int(r[did]))
    vals, prev = [], None
    kn = _col(rows[0], "kernel", "name")
    for r in rows:
        name = r[kn]
        first = name != prev
        prev = name
        if not re.search(kernel_re, name) or (first_of_run and not first):
            continue
        if grid is not None:
            try:
                g = int(r[_col(r, "grid", "size")])
            except KeyError:
                g = None
            if g is not None and g != grid:
                continue
        vals.append(float(r[_col(r, "counter", "value")]))
    if not vals:
        raise SystemExit("no %s rows for /%s/ in %s" % (counter, kernel_re, d))
    return vals


def cmd_summarize_pmc(args):
    copy_kib = args.copy_mib * 1024.0
    cf = statistics.median(_pmc_values(args.copy_fetch, "FETCH_SIZE", args.copy_kernel))
    cw = statistics.median(_pmc_values(args.copy_write, "WRITE_SIZE", args.copy_kernel))
    f_fetch = copy_kib / cf
    f_write = copy_kib / cw
    kf = statistics.median(_pmc_values(args.fetch, "FETCH_SIZE", args.kernel, args.grid,
                                       args.first_of_run))
    kw = statistics.median(_pmc_values(args.write, "WRITE_SIZE", args.kernel, args.grid,
                                       args.first_of_run))
    sys.path.insert(0, ROOT)
    from bench import kernel_source_hash
    out = {
        "kernel": args.kernel,
        "grid_size": args.grid,
        "first_of_run_only": args.first_of_run,
        "kernel_source_hash": kernel_source_hash(),
        "fetch_kib_per_launch_raw": kf,
        "write_kib_per_launch_raw": kw,
        "copy_fetch_kib_raw": cf,
        "copy_write_kib_raw": cw,
        "copy_kib_expected": copy_kib,
        "fetch_scale": f_fetch,
        "write_scale": f_write,
        "bytes_per_launch": kf * f_fetch * 1024.0 + kw * f_write * 1024.0,
        "fetch_bytes_per_launch": kf * f_fetch * 1024.0,
        "write_bytes_per_launch": kw * f_write * 1024.0,
        "commands": args.cmd,
    }
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def _counter_rows(d):
    rows = []
    for path in _find(d, "counter_collection.csv"):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    return rows


def cmd_summarize_counters(args):
    """Counter medians per kernel selection. A selection is
    LABEL|REGEX|GRID|PLACE with GRID an integer or *, and PLACE first (the
    dispatch opens a run of consecutive dispatches of its kernel), later or
    any, with an optional :N that also requires the run to be N long."""
    sels = []
    for s in args.sel:
        label, rx, grid, place = s.split("|")
        sels.append((label, re.compile(rx), None if grid == "*" else int(grid), place))
    table = {}          # (label, counter) -> [values]
    counters = []
    for d in args.dir:
        rows = _counter_rows(d)
        if not rows:
            continue
        did, kn = _col(rows[0], "dispatch", "id"), _col(rows[0], "kernel", "name")
        cn, cv = _col(rows[0], "counter", "name"), _col(rows[0], "counter", "value")
        gcol = None
        try:
            gcol = _col(rows[0], "grid", "size")
        except KeyError:
            pass
        # One entry per dispatch: name, grid, counters.
        disp = {}
        for r in rows:
            e = disp.setdefault(int(r[did]), {"name": r[kn], "grid": r.get(gcol), "c": {}})
            e["c"][r[cn]] = e["c"].get(r[cn], 0.0) + float(r[cv])
        # Runs of consecutive dispatches of one kernel: position and length.
        order = sorted(disp)
        runs, cur = [], []
        for i in order:
            if cur and disp[i]["name"] != disp[cur[-1]]["name"]:
                runs.append(cur)
                cur = []
            cur.append(i)
        if cur:
            runs.append(cur)
        for run in runs:
            for pos, i in enumerate(run):
                disp[i]["first"], disp[i]["run"] = pos == 0, len(run)
        for i in order:
            e = disp[i]
            for label, rx, grid, place in sels:
                if not rx.search(e["name"]):
                    continue
                if grid is not None and e["grid"] is not None and int(e["grid"]) != grid:
                    continue
                kind, _, n = place.partition(":")
                if (kind == "first" and not e["first"]) or (kind == "later" and e["first"]):
                    continue
                if n and e["run"] != int(n):
                    continue
                for c, v in e["c"].items():
                    if c not in counters:
                        counters.append(c)
                    table.setdefault((label, c), []).append(v)
    lines = ["# rocprofv3 counters: %s" % args.title, "", "Command (repo root): `%s`" % args.cmd,
             "", "Median per dispatch (dispatches counted in brackets).", "",
             "| kernel | " + " | ".join(counters) + " |",
             "|---|" + "---:|" * len(counters)]
    for label, _, _, _ in sels:
        cells = []
        for c in counters:
            v = table.get((label, c))
            cells.append("%.4g (%d)" % (statistics.median(v), len(v)) if v else "-")
        lines.append("| %s | %s |" % (label, " | ".join(cells)))
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    p = sub.add_parser("copy")
    p.add_argument("--mib", type=int, default=1024)
    p.add_argument("--reps", type=int, default=5)
    p = sub.add_parser("nkv-sweep")
    p.add_argument("--nkv", default="")
    p.add_argument("--reps", type=int, default=20)
    p = sub.add_parser("balance-probe")
    p.add_argument("--reps", type=int, default=20)
    p = sub.add_parser("summarize-balance")
    p.add_argument("dir")
    p.add_argument("out")
    p.add_argument("--reps", type=int, default=20)
    p.add_argument("--cmd", required=True)
    p.add_argument("--title", default="")
    p = sub.add_parser("summarize-sweep")
    p.add_argument("dir")
    p.add_argument("out")
    p.add_argument("--nkv", default="")
    p.add_argument("--reps", type=int, default=20)
    p.add_argument("--cmd", required=True)
    p.add_argument("--title", default="")
    p = sub.add_parser("summarize-trace")
    p.add_argument("dir")
    p.add_argument("out")
    p.add_argument("--cmd", required=True)
    p.add_argument("--title", default="")
    p = sub.add_parser("summarize-pmc")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel", "--out", "--cmd"):
        p.add_argument(a, required=True)
    p.add_argument("--copy-kernel", default="copyBuffer")
    p.add_argument("--first-of-run", action="store_true")
    p.add_argument("--copy-mib", type=int, default=1024)
    p.add_argument("--grid", type=int, default=None)
    p = sub.add_parser("summarize-counters")
    p.add_argument("--dir", action="append", required=True)
    p.add_argument("--sel", action="append", required=True)
    p.add_argument("--out", required=True)
    p.add_argument("--title", default="")
    p.add_argument("--cmd", required=True)
    args = ap.parse_args()
    {"copy": cmd_copy, "summarize-trace": cmd_summarize_trace,
     "nkv-sweep": cmd_nkv_sweep, "balance-probe": cmd_balance_probe,
     "summarize-balance": cmd_summarize_balance, "summarize-sweep": cmd_summarize_sweep,
     "summarize-pmc": cmd_summarize_pmc,
     "summarize-counters": cmd_summarize_counters}[args.cmd_name](args)


if __name__ == "__main__":
    main()
