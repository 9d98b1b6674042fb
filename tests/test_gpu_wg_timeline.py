"""The timeline build on the GPU: every workgroup of the three attention kernels leaves a record,
its tile count agrees with the oracle's classification of the workload at that kernel's tile
shape, and its four times are in order.  Runs in a child process, because the timeline loads
libflashmask_stamps.so as the library."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import numpy as np
import oracle
from mask_aware_flashattention_amd import wg_timeline
from workloads import configs

w = configs.WORKLOADS["c2c"]
rows = wg_timeline.run("c2c", 2, raw=True)
gv = configs.global_mask(w)
fwd_tiles = int(oracle.classify(*gv, w.nq, 128, 64)["qcnt"].sum()) * w.B * w.H
bwd_tiles = int(oracle.classify(*gv, w.nq, 64, 64)["kcnt"].sum()) * w.B * w.H
want = {"fwd": (w.B * w.H * (w.nq // 128), fwd_tiles), "dq": (w.B * w.H * (w.nq // 128), fwd_tiles),
        "dkdv": (w.B * w.H * (w.nk // 64), bwd_tiles)}
for k, r in rows.items():
    n, tiles = want[k]
    assert r.shape == (n, 8), (k, r.shape)
    assert int(r[:, 5].sum()) == tiles, (k, int(r[:, 5].sum()), tiles)
    live = r[:, 5] > 0
    t0, t1, t2, t3 = (r[live, i] for i in range(4))
    assert (t0 > 0).all() and (t0 <= t1).all() and (t1 <= t2).all() and (t2 <= t3).all(), k
    span = (r[:, 3].max() - r[:, 0].min()) * wg_timeline.TICK_US
    assert 1.0 < span < 10000.0, (k, span)
    print(k, n, tiles, round(float(span), 1), flush=True)
print(wg_timeline.render("c2c", {k: wg_timeline.summarize(r) for k, r in rows.items()}))
"""


def test_timeline_records_every_workgroup():
    from mask_aware_flashattention_amd.wg_timeline import LIB_STAMPS
    if not os.path.exists(LIB_STAMPS):
        pytest.fail(f"{LIB_STAMPS} is not built (python -m mask_aware_flashattention_amd.build --stamps)")
    print("workgroup timeline of c2c in a child process", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, capture_output=True, text=True,
                       timeout=240)
    print(r.stdout[-3000:], flush=True)
    assert r.returncode == 0, r.stderr[-3000:]
