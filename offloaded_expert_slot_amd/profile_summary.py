"""Summaries of rocprofv3 output for the profiles/ folder.

  python -m offloaded_expert_slot_amd.profile_summary trace --stats S.csv --trace T.csv
      --kernel gather_kernel --skip W --take N --command "..." [--title "..."]
    kernel-trace statistics table, plus the average duration of dispatches
    W .. W+N-1 (in launch order) of the named kernel: the benchmark's timed
    phase of that kernel.

  python -m offloaded_expert_slot_amd.profile_summary pmc --csv C.csv [--csv C2.csv ...]
      --kernel gather_kernel --skip W --take N --command "..."
    per-dispatch averages of the counters in rocprofv3 counter-collection CSVs
    over the same dispatch window.
"""
import argparse
import csv
import hashlib
import os
import re
import statistics

FFN_KERNELS = ("gate_up", "down_", "group_pairs", "combine_pairs")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _short(name):
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void at::") or name.startswith("at::"):
        return "torch: " + re.sub(r"<.*", "", name)[:60]
    return re.sub(r"\(.*", "", name)[:90]


def trace(args):
    rows = list(csv.DictReader(open(args.stats)))
    print(f"# {args.title}\n")
    print("Command (run from /tmp with TMPDIR=/tmp, R = repository root):\n")
    print(f"    {args.command}\n")
    print("rocprofv3 kernel-trace statistics (durations in microseconds):\n")
    print("| kernel | calls | total_us | avg_us | min_us | max_us | % |")
    print("|---|---|---|---|---|---|---|")
    for r in rows[:args.top]:
        print(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['TotalDurationNs'])/1e3:.1f} | "
              f"{float(r['AverageNs'])/1e3:.2f} | {float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | "
              f"{float(r['Percentage']):.1f} |")
    disp = [r for r in csv.DictReader(open(args.trace)) if args.kernel in r["Kernel_Name"]]
    disp.sort(key=lambda r: int(r["Start_Timestamp"]))
    sel = disp[args.skip:args.skip + args.take]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel]
    if durs:
        print(f"\nTimed phase of `{args.kernel}`: dispatches {args.skip}..{args.skip + len(sel) - 1} of "
              f"{len(disp)} in launch order: mean {statistics.mean(durs):.2f} us, median "
              f"{statistics.median(durs):.2f} us, min {min(durs):.2f} us, max {max(durs):.2f} us.")


def pmc(args):
    vals = {}
    for f in args.csv:
        rows = [r for r in csv.DictReader(open(f)) if args.kernel in r.get("Kernel_Name", "")]
        ids = sorted({int(r["Dispatch_Id"]) for r in rows})
        keep = set(ids[args.skip:args.skip + args.take])
        for r in rows:
            if int(r["Dispatch_Id"]) in keep:
                vals.setdefault(r["Counter_Name"], {}).setdefault(int(r["Dispatch_Id"]), 0.0)
                vals[r["Counter_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    print(f"Command: {args.command}\n")
    print(f"Counters of `{args.kernel}`, per dispatch, averaged over dispatches {args.skip}..{args.skip + args.take - 1}:\n")
    for c, d in sorted(vals.items()):
        print(f"- {c}: {statistics.mean(d.values()):.1f} (over {len(d)} dispatches)")


def _per_kernel(rows, value, warm):
    """Mean of value(row) per kernel name over each kernel's dispatches after the first `warm`."""
    by = {}
    for r in sorted(rows, key=lambda r: int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0)):
        by.setdefault(_short(r["Kernel_Name"]), []).append(value(r))
    return {k: (len(v), statistics.mean(v[warm:])) for k, v in by.items() if len(v) > warm}


def ffn(args):
    tr = [r for r in csv.DictReader(open(args.trace)) if any(k in r["Kernel_Name"] for k in FFN_KERNELS)]
    dur = _per_kernel(tr, lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3, args.skip)
    counts = {}
    factor = {}
    for name, path, probe in (("FETCH_SIZE", args.fetch, "hbm_read_kernel"), ("WRITE_SIZE", args.write, "FillFunctor<unsigned char>")):
        rows = list(csv.DictReader(open(path)))
        cal = [float(r["Counter_Value"]) for r in rows if probe in r["Kernel_Name"] and int(r["Grid_Size"]) >= 1 << 20]
        factor[name] = (1 << 20) / max(cal)     # KiB the counter reports for 1 GiB moved
        counts[name] = _per_kernel([r for r in rows if any(k in r["Kernel_Name"] for k in FFN_KERNELS)],
                                   lambda r: float(r["Counter_Value"]) * 1024 * factor[name], args.skip)
    print(f"# {args.title}\n")
    print("Commands (run from /tmp with TMPDIR=/tmp and PYTHONPATH = the repository root R), one pass each:\n")
    for c in args.command:
        print(f"    {c}")
    print(f"\nTimed dispatches: every FFN kernel dispatch after the first {args.skip} launches. Counter scale "
          f"factors from the same runs' 1 GiB read (FETCH_SIZE x {factor['FETCH_SIZE']:.2f}) and 1 GiB fill "
          f"(WRITE_SIZE x {factor['WRITE_SIZE']:.2f}).\n")
    print("| kernel | dispatches | mean us | HBM read MB | HBM write MB | read GB/s |")
    print("|---|---|---|---|---|---|")
    tot_us = tot_r = tot_w = 0.0
    for k, (n, us) in dur.items():
        rd = counts["FETCH_SIZE"].get(k, (0, 0.0))[1]
        wr = counts["WRITE_SIZE"].get(k, (0, 0.0))[1]
        tot_us, tot_r, tot_w = tot_us + us, tot_r + rd, tot_w + wr
        print(f"| {k} | {n} | {us:.2f} | {rd / 1e6:.3f} | {wr / 1e6:.3f} | {rd / (us * 1e3):.0f} |")
    print(f"| **all** | | **{tot_us:.2f}** | **{tot_r / 1e6:.3f}** | **{tot_w / 1e6:.3f}** | "
          f"**{tot_r / (tot_us * 1e3):.0f}** |")
    print(f"\nAlgorithmic bytes per launch (distinct experts x bytes per expert): {args.bytes:,}; HBM reads "
          f"{tot_r / args.bytes:.3f}x of them; kernel time summed {tot_us:.2f} us = "
          f"{args.bytes / (tot_us * 1e3):.0f} GB/s of algorithmic bytes.\n")
    src = "offloaded_expert_slot_amd/csrc/k_ffn.hip"
    sha = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
    print(f"traffic {args.key} bytes_per_launch={int(round(tot_r + tot_w))} source={src} sha256={sha}")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    f = sub.add_parser("ffn")
    for a in ("--trace", "--fetch", "--write", "--key", "--title"):
        f.add_argument(a, required=True)
    f.add_argument("--bytes", type=int, required=True)
    f.add_argument("--skip", type=int, default=4)
    f.add_argument("--command", action="append", default=[])
    t = sub.add_parser("trace")
    t.add_argument("--stats", required=True)
    t.add_argument("--trace", required=True)
    t.add_argument("--title", default="Kernel trace")
    t.add_argument("--top", type=int, default=16)
    p = sub.add_parser("pmc")
    p.add_argument("--csv", action="append", required=True)
    for q in (t, p):
        q.add_argument("--kernel", required=True)
        q.add_argument("--skip", type=int, default=0)
        q.add_argument("--take", type=int, default=1 << 30)
        q.add_argument("--command", default="")
    args = ap.parse_args()
    {"trace": trace, "pmc": pmc, "ffn": ffn}[args.mode](args)


if __name__ == "__main__":
    main()
