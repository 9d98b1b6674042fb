"""Workgroup timeline of the three attention kernels on one workload.

Runs the forward and backward calls of a workload through the debug library
``libflashmask_stamps.so`` (built by ``python -m mask_aware_flashattention_amd.build --stamps``;
its kernels are those of ``libflashmask.so`` plus a per-workgroup record, see
``include/flashmask_debug.h``) and summarises, per kernel, the last call's workgroups:

* start -> first tile: from a workgroup's first instruction to its first tile's barrier (its
  block's list and descriptors, the Q / K / V or Q / dO rows of its first tile);
* walk per tile: the tile walk's time divided by its tiles, over all workgroups and by walk
  length;
* walk end -> end: the output stores;
* refill gap: from a workgroup's end to the start of the workgroup that takes its place on the
  same compute unit;
* residency: the share of compute-unit time with 0, 1, 2 or more workgroups resident;
* finish spread: when the compute units and the XCDs finish.

Usage: ``python -m mask_aware_flashattention_amd.wg_timeline [--workload c3] [--calls 20]``
(from the repository root, on a GPU).  The summary is pure host code (``summarize``).
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

TICK_US = 0.01  # s_memrealtime counts at 100 MHz
KERNELS = ("fwd", "dq", "dkdv")
LIB_STAMPS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflashmask_stamps.so")
BINS = ((1, 2), (2, 5), (5, 10), (10, 20), (20, 40), (40, 80), (80, 1 << 30))


def summarize(rows) -> dict:
    """Statistics of one kernel's records: rows [n_workgroups, 8] of unsigned 64-bit words
    {start, first tile, walk done, end, HW_ID | XCC_ID << 32, tiles, -, -} (times in ticks)."""
    r = np.asarray(rows, dtype=np.int64)
    t0, t1, t2, t3, hw, tiles = (r[:, i] for i in range(6))
    base = int(t0.min())
    live = tiles > 0
    pro = (t1 - t0)[live] * TICK_US
    walk = (t2 - t1)[live] * TICK_US
    epi = (t3 - t2)[live] * TICK_US
    cnt = tiles[live]
    held = float((t3 - t0).sum()) * TICK_US
    out = {
        "workgroups": int(len(r)),
        "tiles": int(tiles.sum()),
        "span_us": float(t3.max() - base) * TICK_US,
        "start_to_first_tile_us": float(pro.mean()) if pro.size else 0.0,
        "walk_per_tile_us": float(walk.sum() / cnt.sum()) if cnt.size else 0.0,
        "walk_end_to_end_us": float(epi.mean()) if epi.size else 0.0,
        "share_start": float(pro.sum()) * 1.0 / held if held else 0.0,
        "share_walk": float(walk.sum()) / held if held else 0.0,
        "share_end": float(epi.sum()) / held if held else 0.0,
        "by_walk_length": [],
    }
    for lo, hi in BINS:
        m = (cnt >= lo) & (cnt < hi)
        if m.any():
            out["by_walk_length"].append((lo, hi, int(m.sum()), float(walk[m].sum() / cnt[m].sum())))
    xcc = (hw >> 32) & 0xF
    cu = xcc * 256 + ((hw >> 8) & 0xFF)  # XCC_ID, then CU_ID | SH_ID | SE_ID of HW_ID
    t_end = int(t3.max())
    occ = np.zeros(4)
    gaps, cu_end = [], []
    for c in np.unique(cu):
        idx = np.flatnonzero(cu == c)
        events = sorted([(int(t0[i]), 1) for i in idx] + [(int(t3[i]), -1) for i in idx])
        level, last = 0, base
        for t, step in events:
            occ[min(level, 3)] += t - last
            last, level = t, level + step
        occ[0] += t_end - last
        cu_end.append((int(t3[idx].max()) - base) * TICK_US)
        # a start refills the slot that has been free longest (starts while no slot has been
        # freed yet are the compute unit's first fill, not refills)
        free = []
        for t, step in events:
            if step < 0:
                free.append(t)
            elif free:
                gaps.append((t - free.pop(0)) * TICK_US)
    out["compute_units"] = int(len(cu_end))
    out["residency"] = (occ / occ.sum()).tolist() if occ.sum() else [0.0] * 4
    cu_end = np.asarray(cu_end)
    out["cu_end_us"] = (float(np.percentile(cu_end, 10)), float(np.median(cu_end)),
                        float(cu_end.max()))
    g = np.asarray(gaps)
    out["refill_gap_us"] = (float(np.median(g)), float(g.mean())) if g.size else (0.0, 0.0)
    xe = [float(t3[xcc == x].max() - base) * TICK_US for x in np.unique(xcc)]
    out["xcd_end_us"] = (min(xe), max(xe))
    return out


def render(workload: str, stats: dict) -> str:
    """Markdown table of the three kernels' statistics."""
    names = {"fwd": "forward", "dq": "dQ", "dkdv": "dK/dV"}
    ks = [k for k in KERNELS if k in stats]
    lines = [f"Workgroup timeline, {workload} (last call of each kernel; times in µs)", "",
             "| | " + " | ".join(names[k] for k in ks) + " |",
             "|---|" + "---|" * len(ks)]

    def row(label, fmt):
        lines.append(f"| {label} | " + " | ".join(fmt(stats[k]) for k in ks) + " |")

    row("workgroups / tiles", lambda s: f"{s['workgroups']} / {s['tiles']}")
    row("span", lambda s: f"{s['span_us']:.1f}")
    row("start → first tile (mean)", lambda s: f"{s['start_to_first_tile_us']:.2f}")
    row("walk per tile", lambda s: f"{s['walk_per_tile_us']:.3f}")
    row("walk end → end (mean)", lambda s: f"{s['walk_end_to_end_us']:.2f}")
    row("workgroup time: start / walk / end",
        lambda s: f"{s['share_start']:.3f} / {s['share_walk']:.3f} / {s['share_end']:.3f}")
    row("refill gap (median / mean)",
        lambda s: f"{s['refill_gap_us'][0]:.2f} / {s['refill_gap_us'][1]:.2f}")
    row("CU time with 0 / 1 / 2 / 3+ workgroups",
        lambda s: " / ".join(f"{x:.3f}" for x in s["residency"]))
    row("CU finish (p10 / median / last)", lambda s: " / ".join(f"{x:.1f}" for x in s["cu_end_us"]))
    row("XCD finish (first / last)", lambda s: " / ".join(f"{x:.1f}" for x in s["xcd_end_us"]))
    for lo, hi in BINS:
        label = f"walk per tile, {lo}–{hi - 1} tiles" if hi < (1 << 30) else f"walk per tile, ≥ {lo} tiles"

        def cell(s, lo=lo):
            for a, _, n, v in s["by_walk_length"]:
                if a == lo:
                    return f"{v:.3f} ({n})"
            return "—"
        row(label, cell)
    return "\n".join(lines)


def run(workload: str, calls: int, raw: bool = False) -> dict:
    """Run `calls` forward + backward calls of the workload through the debug library and
    return each kernel's summary (with ``raw``, each kernel's records instead)."""
    from . import _lib
    if not os.path.exists(LIB_STAMPS):
        raise RuntimeError(f"{LIB_STAMPS} is missing: python -m mask_aware_flashattention_amd.build --stamps")
    _lib.load(LIB_STAMPS)
    dbg = ctypes.CDLL(LIB_STAMPS)
    import torch

    from . import api as fm
    from workloads import configs

    w = configs.WORKLOADS[workload]
    if w.dtype != "bf16":
        raise SystemExit("the timeline runs the bf16 workloads")
    dev = torch.device("cuda")
    gv = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in configs.global_mask(w)]
    vec = gv
    if w.key == "c5":
        vec = list(fm.localize(*gv, configs.C5_CHUNK_START, configs.C5_CHUNK_LEN,
                               w.params["global_n"])[:4])
    t = configs.tensors(w)
    q, k, v, do = (t[n].to(dev) for n in ("q", "k", "v", "do"))
    shape = _lib.FmShape(w.B, w.H, w.nq, w.nk, w.d, _lib.FM_BF16)
    ws_f = torch.empty(fm.fwd_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(fm.bwd_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    for _ in range(calls):
        fm.fwd(q, k, v, *vec, w.scale, out=o, lse=lse, workspace=ws_f)
        fm.bwd(q, k, v, o, do, lse, *vec, w.scale, workspace=ws_b, grads=grads)
    torch.cuda.synchronize()
    n_qb = -(-w.nq // 128)
    bn = 64 if w.nq < 65536 else 128
    grids = {"fwd": w.B * w.H * n_qb, "dq": w.B * w.H * n_qb, "dkdv": w.B * w.H * -(-w.nk // bn)}
    stats = {}
    for kname in KERNELS:
        n = grids[kname]
        if n > 1 << 16:
            raise SystemExit(f"{kname}: {n} workgroups, more than the 65536 records")
        buf = np.zeros(n * 8, dtype=np.uint64)
        getter = getattr(dbg, f"flashmask_debug_stamps_{kname}")
        getter.restype = ctypes.c_int
        getter.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
        if getter(buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes) != 0:
            raise RuntimeError(f"flashmask_debug_stamps_{kname} failed")
        rows = buf.reshape(n, 8).astype(np.int64)
        stats[kname] = rows if raw else summarize(rows)
    return stats


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--calls", type=int, default=20, help="forward + backward calls (the last is summarised)")
    a = ap.parse_args(argv)
    print(render(a.workload, run(a.workload, a.calls)), flush=True)


if __name__ == "__main__":
    sys.exit(main())
