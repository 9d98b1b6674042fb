"""Summarise a rocprofv3 results database (rocpd SQLite) into a short markdown table.

Usage: python -m mask_aware_flashattention_amd.rocprof_summary RESULTS_DB [--command "..."]
Prints per-kernel call counts and average / total durations (microseconds).
"""

from __future__ import annotations

import argparse
import sqlite3


def kernel_stats(db_path: str):
    con = sqlite3.connect(db_path)
    rows = con.execute(
        "select name, total_calls, total_duration, average, percentage from top_kernels").fetchall()
    con.close()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--command", default="")
    ap.add_argument("--title", default="rocprofv3 kernel trace")
    a = ap.parse_args()
    print(f"# {a.title}\n")
    if a.command:
        print(f"Command:\n\n```\n{a.command}\n```\n")
    print("| kernel | calls | avg (us) | total (us) | % of GPU time |")
    print("|---|---:|---:|---:|---:|")
    for name, calls, total, avg, pct in kernel_stats(a.db):
        print(f"| `{name}` | {calls} | {avg:.1f} | {total:.1f} | {pct:.1f} |")


if __name__ == "__main__":
    main()
