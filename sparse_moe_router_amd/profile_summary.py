"""Condense a rocprofv3 kernel-stats CSV (--stats --output-format csv) into a
short text table: kernel, calls, average / min / max duration, share."""
from __future__ import annotations

import csv
import sys


def summarize(path: str, top: int = 25) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"{'kernel':<72} {'calls':>7} {'avg_us':>9} {'min_us':>8} {'max_us':>9} {'pct':>6}"]
    for r in rows[:top]:
        out.append(f"{r['Name'][:72]:<72} {int(r['Calls']):>7} {float(r['AverageNs']) / 1e3:>9.2f} "
                   f"{float(r['MinNs']) / 1e3:>8.2f} {float(r['MaxNs']) / 1e3:>9.2f} {float(r['Percentage']):>6.2f}")
    return "\n".join(out)


if __name__ == "__main__":
    print(summarize(sys.argv[1]))
