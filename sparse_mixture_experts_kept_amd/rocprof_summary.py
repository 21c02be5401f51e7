"""Summarise rocprofv3 output databases (rocpd SQLite) per kernel.

    python -m sparse_mixture_experts_kept_amd.rocprof_summary trace DB [DB ...]
        per-kernel calls, total and average duration (us)
    python -m sparse_mixture_experts_kept_amd.rocprof_summary pmc DB [DB ...]
        per-kernel mean value of each collected counter per dispatch
    python -m sparse_mixture_experts_kept_amd.rocprof_summary traffic \
            FETCH_DB WRITE_DB COPY_FETCH_DB COPY_WRITE_DB COPY_BYTES [OUT.json]
        HBM bytes per dispatch of every kernel: FETCH_SIZE and WRITE_SIZE
        (KiB) scaled by what the same counters read for a plain copy of
        COPY_BYTES bytes; OUT.json (optional) also records a hash of each
        kernel's source so that stale figures can be recognised

Kernel names are shortened to the text before the argument list.
"""

from __future__ import annotations

import re
import sqlite3
import sys
from collections import defaultdict


def short(name: str) -> str:
    """Kernel name without return type, anonymous namespace and arguments."""
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", name)


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


def _mean_counter(db, counter):
    vals = defaultdict(list)
    con = sqlite3.connect(db)
    for name, c, value in con.execute("select kernel_name, counter_name, value from counters_collection"):
        if c == counter:
            vals[short(name)].append(value)
    return {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


# Source files each kernel family is compiled from (relative to csrc/).
KERNEL_SOURCES = {
    "grouped_gemm_prefill_kernel": ["gemm_prefill.hip", "common.hpp"],
    "up_decode_kernel": ["gemm_decode.hip", "common.hpp"],
    "down_decode_kernel": ["gemm_decode.hip", "common.hpp"],
    "decode_stream_kernel": ["gemm_decode_stream.hip", "common.hpp"],
    "router": ["router.hip", "permute_dev.hpp", "common.hpp"],
    "route_permute": ["router.hip", "permute_dev.hpp", "common.hpp"],
    "permute_kernel": ["permute.hip", "permute_dev.hpp", "common.hpp"],
    "permute_small_kernel": ["permute.hip", "permute_dev.hpp", "common.hpp"],
    "combine_kernel": ["combine.hip", "common.hpp"],
    "rmsnorm_residual_kernel": ["combine.hip", "common.hpp"],
}


def source_hash(kernel: str):
    """sha256 over the sources a kernel is built from, or None if unknown."""
    import hashlib
    import os

    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    bare = kernel.split("::")[-1] if "<" not in kernel else kernel[: kernel.index("<")].split("::")[-1] + kernel[kernel.index("<"):]
    for prefix, files in KERNEL_SOURCES.items():
        if bare.startswith(prefix):
            h = hashlib.sha256()
            for fn in files:
                with open(os.path.join(csrc, fn), "rb") as fh:
                    h.update(fh.read())
            return h.hexdigest()
    return None


def traffic(args):
    import json

    fetch_db, write_db, copy_fetch_db, copy_write_db, copy_bytes = args[:5]
    out_path = args[5] if len(args) > 5 else None
    copy_bytes = float(copy_bytes)
    fetch, n_fetch = _mean_counter(fetch_db, "FETCH_SIZE")
    write, n_write = _mean_counter(write_db, "WRITE_SIZE")
    cf, _ = _mean_counter(copy_fetch_db, "FETCH_SIZE")
    cw, _ = _mean_counter(copy_write_db, "WRITE_SIZE")
    # The copy probe is the largest kernel in its run.
    f_factor = copy_bytes / (max(cf.values()) * 1024.0)
    w_factor = copy_bytes / (max(cw.values()) * 1024.0)
    print(f"copy probe ({copy_bytes:.0f} B read and written): FETCH_SIZE x{f_factor:.3f}, WRITE_SIZE x{w_factor:.3f}")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read bytes | HBM written bytes |")
    print("|---|---|---|---|---|---|")
    table = {}
    for k in sorted(set(fetch) | set(write)):
        rd = fetch.get(k, 0.0) * 1024.0 * f_factor
        wr = write.get(k, 0.0) * 1024.0 * w_factor
        print(f"| {k} | {n_fetch.get(k, 0)}/{n_write.get(k, 0)} | {fetch.get(k, 0):.6g} | {write.get(k, 0):.6g} "
              f"| {rd:.6g} | {wr:.6g} |")
        table[k] = {"read_bytes": rd, "write_bytes": wr, "source_sha256": source_hash(k)}
    if out_path:
        with open(out_path, "w") as fh:
            json.dump({"fetch_factor": f_factor, "write_factor": w_factor, "kernels": table}, fh, indent=1)


if __name__ == "__main__":
    mode, rest = sys.argv[1], sys.argv[2:]
    {"trace": trace, "pmc": pmc, "traffic": traffic}[mode](rest)
