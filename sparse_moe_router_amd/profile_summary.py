"""Condense rocprofv3 CSV output into short text tables.

  python -m sparse_moe_router_amd.profile_summary stats  <kernel_stats.csv>
      kernel, calls, average / min / max duration, share (--kernel-trace --stats)
  python -m sparse_moe_router_amd.profile_summary counters <counter_collection.csv> [name-substring ...]
      per kernel: dispatches and the mean value of each counter per dispatch (--pmc)
"""
from __future__ import annotations

import csv
import sys
from collections import defaultdict


def summarize(path: str, top: int = 25) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"{'kernel':<72} {'calls':>7} {'avg_us':>9} {'min_us':>8} {'max_us':>9} {'pct':>6}"]
    for r in rows[:top]:
        out.append(f"{r['Name'][:72]:<72} {int(r['Calls']):>7} {float(r['AverageNs']) / 1e3:>9.2f} "
                   f"{float(r['MinNs']) / 1e3:>8.2f} {float(r['MaxNs']) / 1e3:>9.2f} {float(r['Percentage']):>6.2f}")
    return "\n".join(out)


def counter_means(path: str, names=()) -> dict:
    """{(kernel, counter): (dispatches, mean value per dispatch)} for kernels whose name contains any of `names`
    (all kernels if none are given)."""
    acc = defaultdict(lambda: [0, 0.0])
    seen = defaultdict(set)
    for r in csv.DictReader(open(path)):
        k = r["Kernel_Name"]
        if names and not any(n in k for n in names):
            continue
        key = (k, r["Counter_Name"])
        acc[key][1] += float(r["Counter_Value"])
        seen[key].add(r["Dispatch_Id"])
    return {key: (len(seen[key]), v[1] / max(len(seen[key]), 1)) for key, v in acc.items()}


def counters(path: str, names=()) -> str:
    out = [f"{'kernel':<72} {'counter':<12} {'dispatches':>10} {'mean/dispatch':>14}"]
    for (k, c), (n, mean) in sorted(counter_means(path, names).items()):
        out.append(f"{k[:72]:<72} {c:<12} {n:>10} {mean:>14.1f}")
    return "\n".join(out)


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "counters":
        print(counters(sys.argv[2], tuple(sys.argv[3:])))
    elif len(sys.argv) >= 3 and sys.argv[1] == "stats":
        print(summarize(sys.argv[2]))
    else:
        print(summarize(sys.argv[1]))
