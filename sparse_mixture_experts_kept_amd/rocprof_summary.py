"""Summarise rocprofv3 output databases (rocpd SQLite) per kernel.

    python -m sparse_mixture_experts_kept_amd.rocprof_summary trace DB [DB ...]
        per-kernel calls, total and average duration (us)
    python -m sparse_mixture_experts_kept_amd.rocprof_summary pmc DB [DB ...]
        per-kernel mean value of each collected counter per dispatch

Kernel names are shortened to the text before the argument list.
"""

from __future__ import annotations

import re
import sqlite3
import sys
from collections import defaultdict


def short(name: str) -> str:
    name = re.sub(r"\(.*", "", name)
    return name.replace("void ", "")


def trace(dbs):
    rows = defaultdict(list)
    for db in dbs:
        con = sqlite3.connect(db)
        for name, dur in con.execute("select name, duration from kernels"):
            rows[short(name)].append(dur / 1e3)
    out = sorted(rows.items(), key=lambda kv: -sum(kv[1]))
    print("| kernel | calls | total us | avg us | min us | max us |")
    print("|---|---|---|---|---|---|")
    for k, v in out:
        print(f"| {k} | {len(v)} | {sum(v):.1f} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")


def pmc(dbs):
    rows = defaultdict(lambda: defaultdict(list))
    for db in dbs:
        con = sqlite3.connect(db)
        for name, counter, value in con.execute("select kernel_name, counter_name, value from counters_collection"):
            rows[short(name)][counter].append(value)
    counters = sorted({c for v in rows.values() for c in v})
    print("| kernel | dispatches | " + " | ".join(counters) + " |")
    print("|---|---|" + "---|" * len(counters))
    for k, v in sorted(rows.items()):
        n = max(len(x) for x in v.values())
        cells = [f"{sum(v[c]) / len(v[c]):.4g}" if v.get(c) else "" for c in counters]
        print(f"| {k} | {n} | " + " | ".join(cells) + " |")


if __name__ == "__main__":
    mode, dbs = sys.argv[1], sys.argv[2:]
    {"trace": trace, "pmc": pmc}[mode](dbs)
