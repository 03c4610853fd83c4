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
import re
import statistics


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


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
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
    trace(args) if args.mode == "trace" else pmc(args)


if __name__ == "__main__":
    main()
