"""Helpers for the rocprofv3 evidence behind bench.py's roofline figures.

    python bench_profile.py copy [--mib 1024] [--reps 5]
        A plain device-to-device copy of known size (reads and writes MIB
        MiB each per launch): the reference that scales the FETCH_SIZE and
        WRITE_SIZE counters to bytes.
    python bench_profile.py summarize-trace DIR OUT.md --cmd "..."
        Turns a `rocprofv3 --kernel-trace --stats -f csv` directory into a
        short markdown table (calls, average and total time per kernel).
    python bench_profile.py summarize-pmc --fetch DIR --write DIR
            --copy-fetch DIR --copy-write DIR --kernel REGEX --grid N
            --out OUT.json --cmd "..."
        Per-launch HBM bytes of one kernel from FETCH_SIZE / WRITE_SIZE runs,
        each scaled by what the same counter reads for the copy above.
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
    rows = []
    for path in _find(args.dir, "kernel_stats.csv"):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise SystemExit("empty stats")
    kn = _col(rows[0], "name")
    kc = _col(rows[0], "calls")
    kt = _col(rows[0], "totaldurationns")
    ka = _col(rows[0], "averagens")
    lines = ["# rocprofv3 kernel statistics: %s" % args.title, "",
             "Command (repo root): `%s`" % args.cmd, "",
             "| kernel | calls | average (us) | total (ms) |", "|---|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r[kt])):
        name = r[kn]
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append("| `%s` | %s | %.2f | %.3f |" % (name, r[kc], float(r[ka]) / 1e3,
                                                     float(r[kt]) / 1e6))
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _pmc_values(d, counter, kernel_re, grid=None):
    """Counter value per dispatch of kernels matching kernel_re (and grid)."""
    vals = []
    for path in _find(d, "counter_collection.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get(_col(r, "counter", "name")) != counter:
                    continue
                if not re.search(kernel_re, r[_col(r, "kernel", "name")]):
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
    kf = statistics.median(_pmc_values(args.fetch, "FETCH_SIZE", args.kernel, args.grid))
    kw = statistics.median(_pmc_values(args.write, "WRITE_SIZE", args.kernel, args.grid))
    sys.path.insert(0, ROOT)
    from bench import kernel_source_hash
    out = {
        "kernel": args.kernel,
        "grid_size": args.grid,
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


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    p = sub.add_parser("copy")
    p.add_argument("--mib", type=int, default=1024)
    p.add_argument("--reps", type=int, default=5)
    p = sub.add_parser("summarize-trace")
    p.add_argument("dir")
    p.add_argument("out")
    p.add_argument("--cmd", required=True)
    p.add_argument("--title", default="")
    p = sub.add_parser("summarize-pmc")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel", "--out", "--cmd"):
        p.add_argument(a, required=True)
    p.add_argument("--copy-kernel", default="copy|elementwise")
    p.add_argument("--copy-mib", type=int, default=1024)
    p.add_argument("--grid", type=int, default=None)
    args = ap.parse_args()
    {"copy": cmd_copy, "summarize-trace": cmd_summarize_trace,
     "summarize-pmc": cmd_summarize_pmc}[args.cmd_name](args)


if __name__ == "__main__":
    main()
