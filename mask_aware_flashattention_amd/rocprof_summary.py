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

  python -m mask_aware_flashattention_amd.rocprof_summary sweep KERNEL_TRACE_CSV SWEEP_JSON
         [--command C]
      per-size durations of the integer kernels from a kernel trace (``-f csv``) of
      ``bench.py --workload masksweep``: the sweep prints its launch plan in a fixed order, and
      the trace's dispatches of those kernels are matched to it in dispatch order (the first two
      calls of each entry are warm-up); GB/s = the sweep's algorithmic bytes / average duration.

  python -m mask_aware_flashattention_amd.rocprof_summary counters --pmc DB [DB ...]
         --trace DB [--cus 256] [--simds 4] [--ses 32] [--command C]
      per attention kernel: the counters of several --pmc runs (means per dispatch) and the
      kernel's average duration from a kernel trace, with the derived rates: the loaded clock
      (SQ_CYCLES over the shader engines), the fraction of SIMD cycles the matrix core is busy
      (SQ_VALU_MFMA_BUSY_CYCLES), the vector ALU busy and co-issue fractions, instructions per
      MFMA and LDS bytes read per CU and clock.  The kernel-source hashes of the forward and the
      backward are recorded with it.
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


def cmd_workloads(a):
    """Markdown table of `bench.py` JSON lines, one per workload (the benchmark's own HIP-event
    timings; no profiler involved)."""
    print("| workload | U per head | step ms | fwd+bwd TFLOP/s | fwd kernel TFLOP/s | fwd frac | "
          "bwd kernels TFLOP/s | bwd frac | oracle TFLOP/s (cores) |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|---:|")
    with open(a.jsonl) as fh:
        for line in fh:
            if not line.strip():
                continue
            d = json.loads(line)
            c = d["config"]
            u = c.get("unmasked_per_head")
            if "roofline_fwd" in d:
                cb = d.get("cpu_baseline") or {}
                oracle = (f"{cb['value']:.4f} ({cb['cores']})" if "value" in cb else "—")
                print(f"| {c['workload']} | {u:,} | {d['ms_per_step']:.3f} | {d['value']:.1f} | "
                      f"{d['roofline_fwd']['achieved']:.1f} | {d['roofline_fwd']['frac']:.3f} | "
                      f"{d['roofline']['achieved']:.1f} | {d['roofline']['frac']:.3f} | {oracle} |")
            else:  # the all-ranks emulation: whole step only, and one global call beside it
                print(f"| {c['workload']} | {u:,} | {d['ms_per_step']:.3f} | {d['value']:.1f} | — | — "
                      f"| — | — | — (one global call: {d['global_call_ms']:.3f} ms, "
                      f"{d['global_call_tflops']:.1f} TFLOP/s) |")


def cmd_counters(a):
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench  # noqa: E402  (kernel-source hashes)

    vals = {}
    for db in a.pmc:
        con = sqlite3.connect(db)
        acc = {}
        for k, c, v in con.execute("select kernel_name, counter_name, value from counters_collection"):
            acc.setdefault((k, c), []).append(v)
        con.close()
        for (k, c), v in acc.items():
            vals.setdefault(k, {})[c] = sum(v) / len(v)
    durs = {name: avg for name, calls, total, avg, pct in kernel_stats(a.trace)}
    simds = a.cus * a.simds
    print("# Attention kernels: hardware counters at n = 32768 (40 log-normal documents)\n")
    if a.command:
        print(f"Commands:\n\n```\n{a.command}\n```\n")
    print(f"Kernel sources: forward hash `{bench.kernel_source_hash('fwd')}`, backward hash "
          f"`{bench.kernel_source_hash('bwd')}` (code without comments, as the benchmark checks).\n")
    rows = []
    for k, v in sorted(vals.items()):
        if "attn_" not in k:
            continue
        dur = next((d for n, d in durs.items() if n == k), None)
        if dur is None or "SQ_INSTS_MFMA" not in v:
            continue
        cyc = v["SQ_CYCLES"] / a.ses                   # clocks of one shader engine
        clock = cyc / dur * 1e-3                       # GHz (duration in us)
        simd_cycles = simds * cyc
        mfma = v["SQ_INSTS_MFMA"]
        busy = v["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles
        valu = 4 * v["SQ_ACTIVE_INST_VALU"] / simd_cycles
        coex = v["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd_cycles
        rows.append((k, dur, clock, busy, valu, coex, 1 - (busy + valu - coex),
                     v["SQ_INSTS_VALU"] / mfma, v["SQ_INSTS_VALU_TRANS_F32"] / mfma,
                     v["SQ_INSTS_LDS"] / mfma,
                     64 * v["SQ_INSTS_LDS_LOAD_BANDWIDTH"] / (a.cus * cyc),
                     v["SQ_LDS_BANK_CONFLICT"], v.get("SQ_LDS_DATA_FIFO_FULL", 0),
                     mfma * 32768 / (dur * 1e-6) / 1e12))
    print("| kernel | avg (us) | clock (GHz) | MFMA busy | VALU busy | co-issue | neither | "
          "VALU / MFMA | exp / MFMA | LDS instr / MFMA | LDS B/clk/CU | bank conflicts | "
          "LDS data FIFO full | executed MFMA TFLOP/s |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    for r in rows:
        print(f"| `{r[0][:60]}` | {r[1]:.1f} | {r[2]:.2f} | {r[3]:.3f} | {r[4]:.3f} | {r[5]:.3f} | "
              f"{r[6]:.3f} | {r[7]:.2f} | {r[8]:.2f} | {r[9]:.2f} | {r[10]:.1f} | {r[11]:.0f} | "
              f"{r[12]:.3g} | {r[13]:.0f} |")
    print("\nFractions are of SIMD cycles at the loaded clock (MFMA busy counts 32 cycles per "
          "32x32x16 bf16 MFMA; VALU busy from SQ_ACTIVE_INST_VALU; co-issue = cycles with both; "
          "neither = 1 - MFMA - VALU + co-issue).  Executed MFMA TFLOP/s counts every MFMA the "
          "kernel issues (32768 FLOP each), masked entries of listed tiles and the backward's "
          "recomputed products included; it is not the benchmark's useful-FLOP rate.")
    print("\nRaw means per dispatch:\n")
    names = sorted({c for k, v in vals.items() if "attn_" in k for c in v})
    print("| counter | " + " | ".join(f"`{r[0][:40]}`" for r in rows) + " |")
    print("|---|" + "---:|" * len(rows))
    for c in names:
        print(f"| {c} | " + " | ".join(f"{vals[r[0]].get(c, float('nan')):.4g}" for r in rows) + " |")


SWEEP_KERNELS = ("block_minmax_kernel", "classify_kernel", "localize_kernel")


def _trace_rows(csv_path):
    import csv
    with open(csv_path, newline="") as fh:
        rows = list(csv.DictReader(fh))
    out = []
    for r in rows:
        name = r.get("Kernel_Name", "")
        # the block min/max has a vectorised variant for 64- and 128-key blocks
        short = next((k for k in SWEEP_KERNELS if k in name or
                      (k == "block_minmax_kernel" and "block_minmax" in name)), None)
        if short is None:
            continue
        did = int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0)
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3  # ns -> us
        out.append((did, short, dur))
    out.sort()
    return [(k, d) for _, k, d in out]


def cmd_sweep(a):
    rec = json.load(open(a.sweep))
    disp = _trace_rows(a.trace)
    pos = 0
    measured = []
    for entry in rec["plan"]:
        kernels = entry["kernel"].split("+")
        durs = {k: [] for k in kernels}
        for call in range(entry["calls"]):
            for k in kernels:
                if pos >= len(disp) or disp[pos][0] != k:
                    raise SystemExit(f"trace does not follow the plan at dispatch {pos}: "
                                     f"expected {k}, found {disp[pos] if pos < len(disp) else None}")
                if call >= 2:
                    durs[k].append(disp[pos][1])
                pos += 1
        measured.append({k: sum(v) / len(v) for k, v in durs.items()})
    print("# Integer kernels: rocprofv3 kernel-trace durations and HBM throughput\n")
    if a.command:
        print(f"Command:\n\n```\n{a.command}\n```\n")
    print("| kernel | size | algorithmic bytes | avg (us) | GB/s | of 8 TB/s | event-timed GB/s |")
    print("|---|---|---:|---:|---:|---:|---:|")
    res = list(rec["results"])
    k2 = [r for r in res if r["kernel"] == "classify_kernel"]
    k17 = [r for r in res if r["kernel"] != "classify_kernel"]
    i17 = 0
    i2 = 0
    for entry, m in zip(rec["plan"], measured):
        if "workload" not in entry:
            r = k17[i17]
            i17 += 1
            us = m[r["kernel"]]
            size = f"n = 2^{r['n'].bit_length() - 1}"
        elif "classify_kernel" in m:
            r = k2[i2]
            i2 += 1
            us = m["classify_kernel"]
            size = (f"{r['workload']} {r['BM']}x{r['BN']} {r['orientation']}: {r['tiles']} tiles, "
                    f"{r['listed']} listed")
        else:
            continue
        gbs = r["bytes"] / (us * 1e-6) / 1e9
        print(f"| `{r['kernel']}` | {size} | {r['bytes']} | {us:.2f} | {gbs:.1f} | "
              f"{gbs / 8000.0:.3f} | {r['GB/s']} |")


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
    c = sub.add_parser("counters")
    c.add_argument("--pmc", nargs="+", required=True)
    c.add_argument("--trace", required=True)
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--simds", type=int, default=4)
    c.add_argument("--ses", type=int, default=32)
    c.add_argument("--command", default="")
    b = sub.add_parser("workloads")
    b.add_argument("jsonl")
    w = sub.add_parser("sweep")
    w.add_argument("trace")
    w.add_argument("sweep")
    w.add_argument("--command", default="")
    a = ap.parse_args()
    {"kernels": cmd_kernels, "traffic": cmd_traffic, "sweep": cmd_sweep,
     "counters": cmd_counters, "workloads": cmd_workloads}[a.cmd](a)


if __name__ == "__main__":
    main()
