"""Summaries of rocprofv3 output for the profiles/ folder (measurement tooling;
nothing here is on the library's path).

    python -m packed_cache_decode_amd.profile_summary kernels DIR --command "..."
    python -m packed_cache_decode_amd.profile_summary counters DIR --command "..." [--match REGEX]
    python -m packed_cache_decode_amd.profile_summary traffic FETCH_DIR WRITE_DIR --workload W
        --layout L --alg-bytes N --command "..."

DIR is a rocprofv3 output directory written with `-o run --output-format csv`
(run_kernel_stats.csv / run_counter_collection.csv).  `traffic` reads two
counter runs of bench.py (FETCH_SIZE, then WRITE_SIZE) and scales each counter
by what it reads for a kernel of known size in the same run: the library's
streaming-read probe over the 1 GiB flush buffer (FETCH_SIZE) and the device
copy of 256 MiB (WRITE_SIZE); the result is the HBM bytes of one decode
launch (all its kernels), in the format bench.py reads back.
"""

import argparse
import csv
import hashlib
import os
import re
import statistics
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DECODE_KERNELS = re.compile(r"decode_(ring|page|slab|dslab|staged|split|combine|merge|merge_d)_kernel")
STORE_KERNELS = re.compile(r"store(128|_quad)?_kernel")


def short_name(name):
    """Kernel name without argument lists and namespaces."""
    n = name.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    n = n[:cut]
    head, lt, tail = n.partition("<")
    n = head.split("::")[-1] + lt + tail
    if n.startswith("reduce_kernel<512, 1, at::native::ReduceOp<int") and "MaxNan" in name:
        return "torch reduce (amax over the 1 GiB flush buffer)"
    if "FillFunctor" in name:
        return "torch fill (set-up)"
    return n


# kernel sources whose counter-measured HBM traffic a traffic summary records
KERNEL_SOURCES = {
    "decode": ("packed_cache_decode_amd/csrc/tq_decode.hip", "packed_cache_decode_amd/csrc/tq_decode_mfma.hip",
               "packed_cache_decode_amd/csrc/tq_internal.h"),
    "store": ("packed_cache_decode_amd/csrc/tq_store.hip", "packed_cache_decode_amd/csrc/tq_store_common.h",
              "packed_cache_decode_amd/csrc/tq_store_quad.hip", "packed_cache_decode_amd/csrc/tq_internal.h"),
}


def sources_sha256(kind):
    """First 16 hex digits of the SHA-256 of the kernel sources of `kind`."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cmd_kernels(args):
    rows = list(csv.DictReader(open(os.path.join(args.dir, "run_kernel_stats.csv"))))
    print(f"# Kernel trace: {args.title}\n")
    print("Command (from the repository root, `TMPDIR=/tmp`):\n")
    print(f"    {args.command}\n")
    print(f"`run_kernel_stats.csv` of that run ({args.note}):\n")
    print("| kernel | calls | average (us) | min (us) | max (us) |")
    print("|---|---|---|---|---|")
    for r in rows:
        print(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    dec = [r for r in rows if DECODE_KERNELS.search(r["Name"])]
    tot = sum(float(r["AverageNs"]) for r in dec) / 1e3 if dec else None
    if tot is not None:
        print(f"\nDecode kernels, sum of averages: {tot:.2f} us.")
    st = [float(r["AverageNs"]) / 1e3 for r in rows if STORE_KERNELS.search(r["Name"])]
    if args.bench:
        import json
        with open(args.bench) as f:
            b = json.loads(f.read().strip().splitlines()[-1])
        print(f"\nbench.py line of the plain run (no profiler), `{args.bench_command}`:\n")
        keep = {k: b[k] for k in ("value", "unit", "decode_us", "decode_pct_of_hbm_peak", "store_us",
                                  "store_tokens_per_s") if k in b}
        print(f"    {json.dumps(keep)}\n")
        if tot is not None:
            print(f"Event-timed tq_decode there: {b['decode_us']:.2f} us against the kernels' "
                  f"{tot:.2f} us here (the event interval also holds the launch gap between the "
                  f"decode kernels).")
        if st:
            print(f"Event-timed tq_store there: {b['store_us']:.2f} us against the kernel's "
                  f"{st[0]:.2f} us here.")


def _counters(path):
    rows = list(csv.DictReader(open(os.path.join(path, "run_counter_collection.csv"))))
    per = defaultdict(lambda: defaultdict(list))      # kernel -> counter -> [values per dispatch]
    for r in rows:
        per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return per, rows


def cmd_counters(args):
    per, rows = _counters(args.dir)
    pat = re.compile(args.match) if args.match else None
    print(f"# Counters: {args.title}\n")
    print("Command (from the repository root, `TMPDIR=/tmp`):\n")
    print(f"    {args.command}\n")
    print("Per-dispatch medians over the run's launches of each kernel (each counter summed over the "
          "whole device by rocprofv3):\n")
    for k in sorted(per):
        if pat and not pat.search(k):
            continue
        d = per[k]
        n = max(len(v) for v in d.values())
        print(f"## `{short_name(k)}` ({n} dispatches)\n")
        print("| counter | median per dispatch |")
        print("|---|---|")
        for c in sorted(d):
            print(f"| {c} | {statistics.median(d[c]):.6g} |")
        print()


def _per_dispatch(path, counter):
    """{kernel name: [value per dispatch]} for one counter."""
    per, _ = _counters(path)
    return {k: v[counter] for k, v in per.items() if counter in v}


def cmd_traffic(args):
    fetch = _per_dispatch(args.fetch_dir, "FETCH_SIZE")
    write = _per_dispatch(args.write_dir, "WRITE_SIZE")
    gib = 1 << 30
    # calibration: the streaming-read probe reads exactly the 1 GiB flush buffer
    probe = [v for k, vals in fetch.items() if "probe_regs_kernel<false>" in k for v in vals]
    f_factor = gib / (statistics.median(probe) * 1024.0) if probe else 2.0
    # the largest device copy is the 256 MiB copy probe
    copies = [v for k, vals in write.items() if "copyBuffer" in k for v in vals]
    big = max(copies) if copies else None
    w_factor = (256 << 20) / (big * 1024.0) if big else 1.0
    kind = args.kind
    match = DECODE_KERNELS if kind == "decode" else STORE_KERNELS
    total, lines = 0.0, []
    for k in sorted(set(fetch) | set(write)):
        if not match.search(k) or "probe" in k:
            continue
        fk = statistics.median(fetch[k]) if k in fetch else 0.0
        wk = statistics.median(write[k]) if k in write else 0.0
        b_read, b_write = fk * 1024 * f_factor, wk * 1024 * w_factor
        total += b_read + b_write
        lines.append(f"#   {short_name(k)}: FETCH_SIZE {fk:.1f} KiB -> {b_read:.0f} B read; "
                     f"WRITE_SIZE {wk:.1f} KiB -> {b_write:.0f} B written")
    print(f"# HBM traffic of one {kind} launch (all its kernels), workload {args.workload}, "
          f"page layout {args.layout}")
    print("# Two counter runs, one per counter (from the repository root, TMPDIR=/tmp):")
    print(f"#   {args.command}")
    print("# Per-dispatch medians over the run's launches, in KiB, scaled by what the same counter")
    print("# reads for kernels of known size in the same run:")
    print(f"#   FETCH_SIZE: the streaming-read probe over 1 GiB -> factor {f_factor:.4f}")
    print(f"#   WRITE_SIZE: the device copy of 256 MiB -> factor {w_factor:.4f}")
    for ln in lines:
        print(ln)
    print(f"workload: {args.workload}")
    print(f"kernel_sources_sha256: {sources_sha256(kind)}")
    print(f"hbm_bytes_per_launch: {total:.0f}")
    print(f"algorithmic_bytes_per_launch: {args.alg_bytes}")
    print(f"traffic_over_algorithmic: {total / args.alg_bytes:.4f}")


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("dir")
    k.add_argument("--command", required=True)
    k.add_argument("--title", default="bench.py")
    k.add_argument("--note", default="every decode and store dispatch follows a 1 GiB read (cold)")
    k.add_argument("--bench", default=None, help="JSON line of a plain bench.py run to compare with")
    k.add_argument("--bench-command", default="python bench.py")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--command", required=True)
    c.add_argument("--title", default="bench.py")
    c.add_argument("--match", default=None)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--kind", choices=["decode", "store"], default="decode")
    t.add_argument("--workload", required=True)
    t.add_argument("--layout", default="aos")
    t.add_argument("--alg-bytes", type=int, required=True)
    t.add_argument("--command", required=True)
    args = ap.parse_args(argv)
    {"kernels": cmd_kernels, "counters": cmd_counters, "traffic": cmd_traffic}[args.what](args)


if __name__ == "__main__":
    main(sys.argv[1:])
