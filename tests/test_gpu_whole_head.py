"""Full-size parity of whole heads: every query row (O, LSE, dQ) and every key column (dK, dV) of
a head, element by element against the float64 oracle, at the full sizes of the 32K, 128K and
context-parallel workloads and in the launch configuration the benchmark times (the plain
flashmask_fwd / flashmask_bwd calls on contiguous tensors).

The oracle runs its own row functions on exact sub-problems (tests/parity.py,
whole_head_reference): a block of query rows only meets the keys that one of its rows can see,
so the document masks split per document and the sliding window per row block and its window of
keys, and the dense oracle's cost stays within seconds per head.  For the context-parallel share
the oracle takes the *global* vectors at the owned global rows while the GPU runs the localised
ones (Theorem 1 of the explainer's clip-shift-max paragraph, end to end)."""

import numpy as np
import pytest
import torch

import oracle
from tests.parity import (TOL, assert_close, assert_lse, dev_i32, f64, whole_head_reference)
from workloads import configs, masks

pytestmark = pytest.mark.gpu

# workload -> heads compared whole
HEADS = {"c3": (0, 31), "c3m": (0,), "c4swa": (0,), "c4doc": (0,), "c5": (0, 15)}


@pytest.fixture(scope="module")
def fm():
    import mask_aware_flashattention_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("key", sorted(HEADS))
def test_whole_heads(fm, key):
    w = configs.WORKLOADS[key]
    gv = configs.global_mask(w)
    if key == "c5":
        lv = fm.localize(*[dev_i32(x) for x in gv], configs.C5_CHUNK_START, configs.C5_CHUNK_LEN,
                         w.params["global_n"])
        want_v = oracle.localize(*gv, configs.C5_CHUNK_START, configs.C5_CHUNK_LEN,
                                 w.params["global_n"])
        for a, b in zip(lv[:4], want_v[:4]):
            assert np.array_equal(a.cpu().numpy(), b)
        vdev = list(lv[:4])
    else:
        vdev = [dev_i32(x) for x in gv]
    mask_rows = configs.owned_rows(w)
    t = configs.tensors(w)
    qd, kd, vd, dod = (t[n].cuda() for n in ("q", "k", "v", "do"))
    print(f"whole heads {key}: B={w.B} H={w.H} nq={w.nq} nk={w.nk}, heads {HEADS[key]}",
          flush=True)
    o, lse = fm.fwd(qd, kd, vd, *vdev, w.scale)
    dq, dk, dv = fm.bwd(qd, kd, vd, o, dod, lse, *vdev, w.scale)
    torch.cuda.synchronize()
    tol = TOL[w.dtype]
    for h in HEADS[key]:
        q64, k64, v64, do64 = (t[n][0, h].to(torch.float64).numpy() for n in ("q", "k", "v", "do"))
        O, LSE, dQ, dK, dV = whole_head_reference(q64, k64, v64, do64, gv, mask_rows,
                                                  np.float32(w.scale))
        assert_close(f"{key} O h={h}", f64(o[0, h]), O, tol)
        assert_lse(f64(lse[0, h]), LSE)
        assert_close(f"{key} dQ h={h}", f64(dq[0, h]), dQ, tol)
        assert_close(f"{key} dK h={h}", f64(dk[0, h]), dK, tol)
        assert_close(f"{key} dV h={h}", f64(dv[0, h]), dV, tol)
        print(f"  head {h}: all {w.nq} rows and {w.nk} key columns within {tol:.0e}", flush=True)


@pytest.mark.parametrize("family", ["documents", "window"])
def test_whole_heads_fp32(fm, family):
    """The float32 path (d = 64) at a size that spans many tiles in both directions: nq = nk =
    8192 + 37 (ragged last blocks), 12 log-normal causal documents or a 1000-key sliding window,
    both heads of B = 1, H = 2 compared whole (every row of O, LSE and dQ, every key column of
    dK and dV) against the float64 oracle at the float32 bar."""
    n, H, d = 8192 + 37, 2, 64
    r = np.random.default_rng(np.random.SeedSequence([8229, 64, 0 if family == "documents" else 1]))
    if family == "documents":
        vec = masks.document(n, masks.lognormal_lengths(r, n, 12))
    else:
        vec = masks.sliding_window(n, 1000)
    q, k, v = (r.standard_normal((1, H, n, d)).astype(np.float32) for _ in range(3))
    do = (0.5 * r.standard_normal((1, H, n, d))).astype(np.float32)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    print(f"whole heads fp32 {family}: n={n} H={H} d={d}", flush=True)
    qd, kd, vd, dod = (torch.from_numpy(x).cuda() for x in (q, k, v, do))
    vdev = [dev_i32(x) for x in vec]
    o, lse = fm.fwd(qd, kd, vd, *vdev, scale)
    dq, dk, dv = fm.bwd(qd, kd, vd, o, dod, lse, *vdev, scale)
    torch.cuda.synchronize()
    tol = TOL["fp32"]
    for h in range(H):
        O, LSE, dQ, dK, dV = whole_head_reference(
            q[0, h].astype(np.float64), k[0, h].astype(np.float64), v[0, h].astype(np.float64),
            do[0, h].astype(np.float64), vec, np.arange(n), np.float32(scale))
        assert_close(f"fp32 {family} O h={h}", f64(o[0, h]), O, tol)
        assert_lse(f64(lse[0, h]), LSE)
        assert_close(f"fp32 {family} dQ h={h}", f64(dq[0, h]), dQ, tol)
        assert_close(f"fp32 {family} dK h={h}", f64(dk[0, h]), dK, tol)
        assert_close(f"fp32 {family} dV h={h}", f64(dv[0, h]), dV, tol)
        print(f"  head {h}: all {n} rows and key columns within {tol:.0e}", flush=True)
