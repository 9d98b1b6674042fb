"""Benchmark: mask-aware attention forward + backward on one MI355X.

One step = one pass of the whole path over the workload: flashmask_fwd (block min/max,
classification, block order, attention forward) then flashmask_bwd (the same at both tile
shapes, dQ kernel, which also writes -D and LSE*log2e per row, then the dK/dV kernel); for the context-parallel share the step also
starts with flashmask_localize.  ``--workload cp16`` times all 16 ranks of the 128K
context-parallel share one after another on this GPU (per rank: localize, prune list, forward,
backward on its 8192 rows against all 131072 keys) beside one global call.  Inputs are seeded synthetic tensors resident in HBM before the
timed region.  Throughput counts unmasked score entries only: 4*d FLOPs per entry forward,
10*d backward.

Prints one JSON line.  ``--gpus`` above 1 is refused: this build runs on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
METRIC = "achieved TFLOP/s (unmasked FLOPs) fwd & bwd, % of bf16 MFMA peak, 1 GPU"
TRAFFIC_FILES = {"bwd": os.path.join(ROOT, "profiles", "attn_bwd_c3_hbm_traffic.txt"),
                 "fwd": os.path.join(ROOT, "profiles", "attn_fwd_c3_hbm_traffic.txt")}
KERNEL_SOURCES = {"bwd": ["attn_bwd.hip", "attn_bwd_dq.hip", "fm_common.hpp", "launch.hpp"],
                  "fwd": ["attn_fwd.hip", "fm_common.hpp", "launch.hpp"]}


def unmasked_entries(vectors, nq: int) -> int:
    """Unmasked (row, key) entries of one head: nq per key minus the union of the key's two
    closed stretches clipped to [0, nq)."""
    import numpy as np
    a1, b1, a2, b2 = (np.clip(np.asarray(v, dtype=np.int64), 0, nq) for v in vectors)
    l1 = np.maximum(b1 - a1, 0)
    l2 = np.maximum(b2 - a2, 0)
    both = (l1 > 0) & (l2 > 0)
    ov = np.where(both, np.maximum(np.minimum(b1, b2) - np.maximum(a1, a2), 0), 0)
    return int(nq * len(a1) - (l1 + l2 - ov).sum())


def code_text(src: str) -> str:
    """A kernel source without its comments, trailing blanks and empty lines: the text whose
    change can change the kernel (the sources hold no string with a comment marker in it)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in src.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash(which: str = "bwd") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[which]:
        with open(os.path.join(ROOT, "mask_aware_flashattention_amd", "csrc", f)) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(which: str):
    """HBM bytes per launch of the forward attention kernel, or of the backward's two kernels
    together, at the n=32768 workload,
    from the committed counter summary, or None if it is missing or was taken on different
    kernel sources."""
    path = TRAFFIC_FILES[which]
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash(which):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, vectors, tensors, mask_rows, seconds: float):
    """The float64 oracle, as it stands, on a bounded sample of the same workload: forward and
    backward for growing blocks of query rows of head 0 until one run takes >= ``seconds``."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    cores = len(os.sched_getaffinity(0))
    q = tensors["q"][:, :1]
    k, v, do = tensors["k"][:, :1], tensors["v"][:, :1], tensors["do"][:, :1]
    scale = np.float32(w.scale)
    rows_n = 64
    rng = np.random.default_rng(0)
    last = None
    with threadpool_limits(limits=1):
        while True:
            start = int(rng.integers(0, max(1, w.nq - rows_n)))
            sel = np.arange(start, min(w.nq, start + rows_n))
            t0 = time.perf_counter()
            oracle.attention_fwd(q[:, :, sel], k, v, vectors, scale, row_block=16, workers=cores,
                                 rows=mask_rows[sel])
            oracle.attention_bwd(q[:, :, sel], k, v, do[:, :, sel], vectors, scale, row_block=16,
                                 workers=cores, rows=mask_rows[sel])
            dt = time.perf_counter() - t0
            M = oracle.dense_mask(*vectors, mask_rows[sel])
            u = int((~M).sum())
            last = (dt, u, len(sel))
            if dt >= seconds or rows_n >= w.nq:
                break
            rows_n = min(w.nq, max(rows_n * 2, int(rows_n * seconds / max(dt, 1e-3) * 1.1)))
    dt, u, nrows = last
    flops = 14 * w.d * u
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"head 0, {nrows} consecutive query rows of {w.nq}: float64 dense forward + "
                   f"backward against all {w.nk} keys, {dt:.1f} s; throughput counts the "
                   f"sample's {u} unmasked entries at 14*d FLOPs each"),
        "seconds": dt,
        "host": host_info(),
    }


def host_info():
    """The CPU model and the numpy / BLAS builds the CPU baseline ran on."""
    import platform

    import numpy as np
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
                       if i.get("user_api") == "blas"})
    except Exception:  # threadpoolctl missing or unable to inspect: leave the BLAS field empty
        blas = []
    return {"cpu_model": model, "numpy": np.__version__, "blas": blas}


def cp_emulation(args):
    """All ranks of the 16-way context-parallel 128K document share, one after another on one
    GPU; value = the global problem's unmasked FLOPs / time of the 16 rank steps."""
    import numpy as np
    import torch

    import mask_aware_flashattention_amd as fm
    from workloads import configs

    fm.load_library()
    dev = torch.device("cuda:0")
    w = configs.WORKLOADS["c5"]
    R, L = configs.C5_DEGREE, configs.C5_CHUNK
    n, H, d = 2 * R * L, w.H, w.d
    gv = configs.global_mask(w)
    gdev = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in gv]
    U = unmasked_entries(gv, n)
    flop = 14 * d * H * U
    g = torch.Generator(device=dev).manual_seed(20261203)
    q, k, v, do = (torch.randn((1, H, n, d), generator=g, device=dev).to(torch.bfloat16)
                   for _ in range(4))
    ranks = []
    for r in range(R):
        starts, lens = [r * L, (2 * R - 1 - r) * L], [L, L]
        rows = torch.cat([torch.arange(a, a + b, device=dev) for a, b in zip(starts, lens)])
        ranks.append((starts, lens, q.index_select(2, rows).contiguous(),
                      do.index_select(2, rows).contiguous()))

    def rank_steps():
        for starts, lens, q_l, do_l in ranks:
            lv = fm.localize(*gdev, starts, lens, n)
            fm.prune_chunks(*lv[:4], lv[4], L, L)
            o_l, lse_l = fm.fwd(q_l, k, v, *lv[:4])
            fm.bwd(q_l, k, v, o_l, do_l, lse_l, *lv[:4])

    def global_step():
        o, lse = fm.fwd(q, k, v, *gdev)
        fm.bwd(q, k, v, o, do, lse, *gdev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    ms_ranks = timed(rank_steps)
    ms_global = timed(global_step)
    print(json.dumps({
        "metric": METRIC, "value": round(flop / (ms_ranks * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_ranks, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "cp16: 16 ranks x 8192 rows of the 131072-row 24-document mask, "
                               "run one after another", "B": 1, "H": H, "n": n, "d": d,
                   "unmasked_per_head": U, "flop_fwd_plus_bwd": flop},
        "global_call_ms": round(ms_global, 4),
        "global_call_tflops": round(flop / (ms_global * 1e-3) / 1e12, 2),
    }), flush=True)


MASK_SWEEP_EXPONENTS = tuple(range(20, 27))  # n = 2^20 .. 2^26 keys
MASK_SWEEP_REPS = 20


def mask_kernel_sweep(args):
    """HBM throughput of the integer kernels on their own, timed with HIP events on the launch
    stream: block min/max (K1: 16 B read per key, 32 B written per key block of 64) and
    clip-shift-max localisation (K7: 16 B read + 16 B written per key; the CP share's two
    chunks of 4096 rows) at n = 2^20 .. 2^26, and tile classification with list compaction (K2)
    at the 128K tile grids.  Every call goes through the C ABI; the launch order is fixed and
    printed in `plan`, so a rocprofv3 kernel trace of this run can be matched dispatch by
    dispatch (``rocprof_summary sweep``)."""
    import ctypes

    import numpy as np
    import torch

    import mask_aware_flashattention_amd as fm
    from mask_aware_flashattention_amd import _lib
    from workloads import configs, masks

    lib = fm.load_library()
    dev = torch.device("cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)
    reps = args.steps if args.steps != 20 else MASK_SWEEP_REPS
    plan, results = [], []

    def timed(fn, n_calls):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_calls):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n_calls

    for e in MASK_SWEEP_EXPONENTS:
        n = 1 << e
        # sliding-window vectors at this length (any values do: the kernels are data-oblivious
        # except for the list lengths, which K1 and K7 do not produce)
        vec = [torch.from_numpy(x).to(dev) for x in masks.sliding_window(n, 4096)]
        out = [torch.empty_like(x) for x in vec]
        BN = 64
        n_kb = -(-n // BN)
        ws = torch.empty(lib.flashmask_classify_workspace_bytes(n, BN), dtype=torch.uint8,
                         device=dev)

        def k1():
            # all outputs NULL: only the block min/max kernel runs (one query block, so the
            # tile-count limit does not apply)
            st = lib.flashmask_classify(*[P(x) for x in vec], n, n, n, BN, P(None), P(None),
                                        P(None), P(None), P(None), P(ws), ws.numel(), stream)
            assert st == 0, st
        starts = (ctypes.c_int32 * 2)(*[c * n // 32 for c in configs.C5_CHUNKS])
        lens = (ctypes.c_int32 * 2)(n // 32, n // 32)
        n_local = ctypes.c_int32()

        def k7():
            st = lib.flashmask_localize(*[P(x) for x in vec], n, n, starts, lens, 2,
                                        *[P(x) for x in out], ctypes.byref(n_local), stream)
            assert st == 0, st
        for name, fn, nbytes in (("block_minmax_kernel", k1, 16 * n + 32 * n_kb),
                                 ("localize_kernel", k7, 32 * n)):
            plan.append({"kernel": name, "n": n, "calls": 2 + reps})
            t = timed(fn, reps)
            results.append({"kernel": name, "n": n, "bytes": nbytes, "us": round(t * 1e6, 3),
                            "GB/s": round(nbytes / t / 1e9, 1),
                            "frac_of_hbm_peak": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)})
        del vec, out, ws

    # K2 at the 128K grids: row lists at the forward tiles (128 x 64) and column lists at the
    # 8-wave backward tiles (64 x 128), both 128K masks.
    for key in ("c4swa", "c4doc"):
        w = configs.WORKLOADS[key]
        vec = [torch.from_numpy(x).to(dev) for x in configs.global_mask(w)]
        for BM, BN, rows in ((128, 64, True), (64, 128, False)):
            n_qb, n_kb = -(-w.nq // BM), -(-w.nk // BN)
            ws = torch.empty(lib.flashmask_classify_workspace_bytes(w.nk, BN), dtype=torch.uint8,
                             device=dev)
            cnt = torch.empty(n_qb if rows else n_kb, dtype=torch.int32, device=dev)
            lst = torch.empty(n_qb * n_kb, dtype=torch.int32, device=dev)
            args_q = (P(cnt), P(lst), P(None), P(None)) if rows else (P(None), P(None), P(cnt),
                                                                       P(lst))

            def k12():
                st = lib.flashmask_classify(*[P(x) for x in vec], w.nq, w.nk, BM, BN, P(None),
                                            *args_q, P(ws), ws.numel(), stream)
                assert st == 0, st

            def k1only():
                st = lib.flashmask_classify(*[P(x) for x in vec], w.nq, w.nk, BM, BN, P(None),
                                            P(None), P(None), P(None), P(None), P(ws), ws.numel(),
                                            stream)
                assert st == 0, st
            plan.append({"kernel": "block_minmax_kernel+classify_kernel", "workload": key,
                         "BM": BM, "BN": BN, "orientation": "rows" if rows else "columns",
                         "calls": 2 + reps})
            t12 = timed(k12, reps)
            plan.append({"kernel": "block_minmax_kernel", "workload": key, "BM": BM, "BN": BN,
                         "calls": 2 + reps})
            t1 = timed(k1only, reps)
            listed = int(cnt.sum())
            nbytes = 32 * n_kb + 4 * (listed + cnt.numel())  # table once, lists and counts
            t2 = max(t12 - t1, 1e-9)
            results.append({"kernel": "classify_kernel", "workload": key, "BM": BM, "BN": BN,
                            "orientation": "rows" if rows else "columns",
                            "tiles": n_qb * n_kb, "listed": listed, "bytes": nbytes,
                            "us": round(t2 * 1e6, 3), "GB/s": round(nbytes / t2 / 1e9, 1),
                            "Gtiles/s": round(n_qb * n_kb / t2 / 1e9, 2)})
    print(json.dumps({"metric": "integer kernels: HBM GB/s (algorithmic bytes / event time)",
                      "unit": "GB/s", "peak_GB/s": PEAK_HBM_GBS, "reps": reps,
                      "results": results, "plan": plan}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB "
                         "(a known-size kernel for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(no collectives or cross-GPU sharding in this build)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mask_aware_flashattention_amd as fm
    from mask_aware_flashattention_amd import _lib
    from workloads import configs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload == "cp16":
        cp_emulation(args)
        return
    if args.workload == "masksweep":
        mask_kernel_sweep(args)
        return
    lib = fm.load_library()
    dev = torch.device("cuda:0")
    w = configs.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        print("bench workloads are bf16", file=sys.stderr)
        sys.exit(1)

    gv = configs.global_mask(w)
    gdev = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in gv]
    localize_args = None
    if w.key == "c5":
        localize_args = (configs.C5_CHUNK_START, configs.C5_CHUNK_LEN, w.params["global_n"])
        vdev = list(fm.localize(*gdev, *localize_args)[:4])
        mask_rows = configs.owned_rows(w)
        vec_cpu_local = [x.cpu().numpy() for x in vdev]
    else:
        vdev = gdev
        mask_rows = np.arange(w.nq)
        vec_cpu_local = gv
    U = unmasked_entries(vec_cpu_local, w.nq)
    flop_f = 4 * w.d * w.B * w.H * U
    flop_b = 10 * w.d * w.B * w.H * U

    t_cpu = configs.tensors(w)
    q, k, v, do = (t_cpu[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    shape = _lib.FmShape(w.B, w.H, w.nq, w.nk, w.d, _lib.FM_BF16)
    ws_f = torch.empty(fm.fwd_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(fm.bwd_workspace_bytes(shape), dtype=torch.uint8, device=dev)

    def step():
        if localize_args is not None:
            fm.localize(*gdev, *localize_args)
        fm.fwd(q, k, v, *vdev, w.scale, out=o, lse=lse, workspace=ws_f)
        fm.bwd(q, k, v, o, do, lse, *vdev, w.scale, workspace=ws_b, grads=(dq, dk, dv))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-step events: call boundaries (current stream) and the attention kernels alone
    mk = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[mk() for _ in range(7)] for _ in range(args.steps)]
    for row in ev:
        for e in row:
            e.record()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for s in range(args.steps):
        e = ev[s]
        lib.flashmask_set_profile_events(e[3].cuda_event, e[4].cuda_event, e[5].cuda_event,
                                         e[6].cuda_event)
        e[0].record()
        if localize_args is not None:
            fm.localize(*gdev, *localize_args)
        fm.fwd(q, k, v, *vdev, w.scale, out=o, lse=lse, workspace=ws_f)
        e[1].record()
        fm.bwd(q, k, v, o, do, lse, *vdev, w.scale, workspace=ws_b, grads=(dq, dk, dv))
        e[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lib.flashmask_set_profile_events(None, None, None, None)

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()

    ms = lambda a, b: float(np.mean([r[a].elapsed_time(r[b]) for r in ev]))
    fwd_call_ms, bwd_call_ms = ms(0, 1), ms(1, 2)
    fwd_kernel_ms, bwd_kernel_ms = ms(3, 4), ms(5, 6)
    ms_per_step = wall * 1e3 / args.steps
    value = (flop_f + flop_b) / (ms_per_step * 1e-3) / 1e12

    on_c3 = w.key == "c3"
    traffic = load_traffic("bwd") if on_c3 else None
    traffic_f = load_traffic("fwd") if on_c3 else None
    bwd_achieved = flop_b / (bwd_kernel_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "nq": w.nq, "nk": w.nk, "d": w.d,
                   "mask": w.family, "unmasked_per_head": U,
                   "flop_fwd": flop_f, "flop_bwd": flop_b},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"call_ms": round(fwd_call_ms, 4), "kernel_ms": round(fwd_kernel_ms, 4),
                "tflops_call": round(flop_f / fwd_call_ms / 1e9, 2),
                "frac_of_peak_call": round(flop_f / fwd_call_ms / 1e9 / PEAK_BF16_TFLOPS, 4)},
        "bwd": {"call_ms": round(bwd_call_ms, 4), "kernel_ms": round(bwd_kernel_ms, 4),
                "tflops_call": round(flop_b / bwd_call_ms / 1e9, 2),
                "frac_of_peak_call": round(flop_b / bwd_call_ms / 1e9 / PEAK_BF16_TFLOPS, 4)},
        # the backward's two kernels (dK/dV, then dQ) run back to back and are timed as one span
        "roofline": {"kernel": "attn_dq_kernel<bf16,128> + attn_bwd_kernel<bf16,128>",
                     "bound": "mfma",
                     "achieved": round(bwd_achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(bwd_achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "roofline_fwd": {"kernel": "attn_fwd_kernel<bf16,128>", "bound": "mfma",
                         "achieved": round(flop_f / (fwd_kernel_ms * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flop_f / (fwd_kernel_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_f},
    }
    if not args.no_cpu_baseline:
        # the oracle takes the global vectors with the global row number of every local row
        out["cpu_baseline"] = cpu_baseline(w, gv, t_cpu, mask_rows, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
