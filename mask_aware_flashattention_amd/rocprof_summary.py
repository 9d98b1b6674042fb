"""Summaries of rocprofv3 results databases (rocpd SQLite) for the committed profiles.

  python -m mask_aware_flashattention_amd.rocprof_summary kernels RESULTS_DB [--title T] [--command C]
      per-kernel call counts and average / total durations (microseconds), as markdown.

  python -m mask_aware_flashattention_amd.rocprof_summary traffic --fetch DB --write DB
         --kernel SUBSTR [SUBSTR ...] --copy-mib N [--command C]
      HBM bytes per launch of one kernel (or the sum over several kernels that together make
      one call, e.g. the backward's dK/dV and dQ kernels) from a FETCH_SIZE run and a
      WRITE_SIZE run, each scaled
      by what the same counter reads for the plain device copy of N MiB that the benchmark runs
      with --calibration-copy-mib N (known bytes / counter bytes).  Prints one JSON object that
      also records the hash of the kernel sources, so the benchmark can tell when the counters
      no longer describe the current kernel.
"""

from __future__ import annotations

import argparse
import json
import os
import sqlite3
import sys

COPY_KERNEL = "copyBuffer"


def kernel_stats(db_path: str):
    con = sqlite3.connect(db_path)
    rows = con.execute(
        "select name, total_calls, total_duration, average, percentage from top_kernels").fetchall()
    con.close()
    return rows


def counter_means(db_path: str, counter: str):
    """{kernel name: mean counter value per dispatch} for one counter."""
    con = sqlite3.connect(db_path)
    acc = {}
    for name, val in con.execute(
            "select kernel_name, value from counters_collection where counter_name = ?", (counter,)):
        acc.setdefault(name, []).append(val)
    con.close()
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _pick(means, substr):
    hits = [k for k in means if substr in k]
    if len(hits) != 1:
        raise SystemExit(f"kernel '{substr}' matches {len(hits)} kernels: {hits}")
    return means[hits[0]]


def cmd_kernels(a):
    print(f"# {a.title}\n")
    if a.command:
        print(f"Command:\n\n```\n{a.command}\n```\n")
    print("| kernel | calls | avg (us) | total (us) | % of GPU time |")
    print("|---|---:|---:|---:|---:|")
    for name, calls, total, avg, pct in kernel_stats(a.db):
        print(f"| `{name}` | {calls} | {avg:.1f} | {total:.1f} | {pct:.1f} |")


def cmd_traffic(a):
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench  # noqa: E402  (for the kernel-source hash the benchmark checks)

    fetch = counter_means(a.fetch, "FETCH_SIZE")
    write = counter_means(a.write, "WRITE_SIZE")
    copy_bytes = a.copy_mib * (1 << 20)
    f_copy, w_copy = _pick(fetch, COPY_KERNEL), _pick(write, COPY_KERNEL)
    f_factor = copy_bytes / (f_copy * 1024.0)
    w_factor = copy_bytes / (w_copy * 1024.0)
    f_k = sum(_pick(fetch, k) for k in a.kernel)
    w_k = sum(_pick(write, k) for k in a.kernel)
    rec = {
        "kernel": " + ".join(a.kernel),
        "fetch_kib_per_launch": f_k,
        "write_kib_per_launch": w_k,
        "copy_mib": a.copy_mib,
        "fetch_scale": round(f_factor, 4),
        "write_scale": round(w_factor, 4),
        "hbm_bytes_per_launch": int(round(f_k * 1024 * f_factor + w_k * 1024 * w_factor)),
        "hbm_read_bytes_per_launch": int(round(f_k * 1024 * f_factor)),
        "hbm_write_bytes_per_launch": int(round(w_k * 1024 * w_factor)),
        "kernel_source_hash": bench.kernel_source_hash(a.sources),
        "command": a.command,
    }
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("db")
    k.add_argument("--title", default="rocprofv3 kernel trace")
    k.add_argument("--command", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True, nargs="+")
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--sources", default="bwd", choices=["bwd", "fwd"])
    t.add_argument("--command", default="")
    a = ap.parse_args()
    {"kernels": cmd_kernels, "traffic": cmd_traffic}[a.cmd](a)


if __name__ == "__main__":
    main()
