"""GPU parity on the five workloads at full size, in the launch configuration the benchmark times.

The tiny fp32 workload is compared element by element with the full oracle.  For the others the
oracle computes sampled query rows (O, LSE, dQ) and sampled key columns (dK, dV) exactly, and
properties that hold at any size are checked on every output:
    sum_j dK_j = 0            (each row's softmax is shift invariant, so sum_j dS_ij = 0)
    sum_j dV_j = sum_i dO_i   over rows that are not fully masked (each row's P sums to 1)
    no NaN anywhere; LSE = -inf exactly on fully masked rows.
The context-parallel share first checks the localised vectors bit-exactly, then compares the
local rows with the oracle run on the *global* mask at the owned global rows (Theorem 1 end to
end)."""

import numpy as np
import pytest
import torch

import oracle
from tests.parity import (TOL, assert_close, assert_lse, cols_reference, dev_i32, f64,
                          rows_reference)
from workloads import configs

pytestmark = pytest.mark.gpu

KEYS = ["c1", "c2a", "c2b", "c2c", "c2d", "c2e", "c2f", "c3", "c3m", "c4swa", "c4doc", "c5"]


@pytest.fixture(scope="module")
def fm():
    import mask_aware_flashattention_amd as m
    m.load_library()
    return m


def rng(*k):
    return np.random.default_rng(np.random.SeedSequence([44, *k]))


def pick_rows(r, nq, vectors, n=40):
    bounds = np.unique(np.clip(np.concatenate([np.asarray(vectors[0]), [0, nq]]), 0, nq))
    special = [0, 1, nq - 1] + list(bounds[(bounds > 0) & (bounds < nq)][:6])
    special += [b - 1 for b in special if 0 < b]
    rand = r.choice(nq, size=min(nq, n), replace=False)
    return np.unique(np.clip(np.concatenate([special, rand]), 0, nq - 1)).astype(np.int64)


def pick_cols(r, nk, vectors, mask_rows, max_rows, n=8):
    tail = r.integers(max(0, nk - 2 * max_rows), nk, size=64)
    cand = np.concatenate([[0, nk - 1], r.permutation(nk)[:256], tail])
    out = []
    for c in cand:
        cnt = int((~oracle.dense_mask(*[np.asarray(x)[[c]] for x in vectors], mask_rows)).sum())
        if 0 < cnt <= max_rows and c not in out:
            out.append(int(c))
        if len(out) >= n:
            break
    return np.array(sorted(out), dtype=np.int64)


def check_invariants(dk, dv, do, lse):
    """Per (b, h) and per feature column, on the full bf16/fp32 outputs."""
    dk64, dv64, do64 = f64(dk), f64(dv), f64(do)
    live = np.isfinite(f64(lse))
    for b in range(dk64.shape[0]):
        for h in range(dk64.shape[1]):
            s = dk64[b, h].sum(0)
            bound = 1e-2 * np.abs(dk64[b, h]).sum(0) + 1e-2
            assert (np.abs(s) <= bound).all(), f"sum dK != 0 (b={b}, h={h}): {np.abs(s).max():.3e}"
            want = do64[b, h][live[b, h]].sum(0)
            bound = 1e-2 * np.abs(dv64[b, h]).sum(0) + 1e-2
            err = np.abs(dv64[b, h].sum(0) - want)
            assert (err <= bound).all(), f"sum dV != sum dO (b={b}, h={h}): {err.max():.3e}"


@pytest.mark.parametrize("key", KEYS)
def test_workload_parity(fm, key):
    w = configs.WORKLOADS[key]
    print(f"workload {key}: {w.name}", flush=True)
    gv = configs.global_mask(w)
    if key == "c5":
        gdev = [dev_i32(x) for x in gv]
        out = fm.localize(*gdev, configs.C5_CHUNK_START, configs.C5_CHUNK_LEN, w.params["global_n"])
        torch.cuda.synchronize()
        want = oracle.localize(*gv, configs.C5_CHUNK_START, configs.C5_CHUNK_LEN,
                               w.params["global_n"])
        assert out[4] == want[4] == w.nq
        for a, b in zip(out[:4], want[:4]):
            assert np.array_equal(a.cpu().numpy(), b)
        vdev = list(out[:4])
        mask_rows_all = configs.owned_rows(w)     # global row of each local row
    else:
        vdev = [dev_i32(x) for x in gv]
        mask_rows_all = np.arange(w.nq)

    t = configs.tensors(w)
    qd, kd, vd, dod = (t[n].cuda() for n in ("q", "k", "v", "do"))
    print(f"  fwd+bwd on GPU B={w.B} H={w.H} nq={w.nq} nk={w.nk} d={w.d} {w.dtype}", flush=True)
    o, lse = fm.fwd(qd, kd, vd, *vdev, w.scale)
    dq, dk, dv = fm.bwd(qd, kd, vd, o, dod, lse, *vdev, w.scale)
    torch.cuda.synchronize()
    for name, x in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert not torch.isnan(x).any(), f"NaN in {name}"
    tol = TOL[w.dtype]
    scale = np.float32(w.scale)

    if key == "c1":
        O, LSE = oracle.attention_fwd(t["q"], t["k"], t["v"], gv, scale)
        dQ, dK, dV = oracle.attention_bwd(t["q"], t["k"], t["v"], t["do"], gv, scale)
        assert_close("O", f64(o), O, tol)
        assert_lse(f64(lse), LSE)
        assert_close("dQ", f64(dq), dQ, tol)
        assert_close("dK", f64(dk), dK, tol)
        assert_close("dV", f64(dv), dV, tol)
        return

    check_invariants(dk, dv, dod, lse)
    r = rng(KEYS.index(key))
    heads = sorted({0, w.H - 1})
    # bound the oracle's work per sampled column (rows attending it x keys those rows see)
    max_rows = 8192 if w.nk <= 8192 else (4096 if w.family == "sliding_window" else 768)
    for h in heads:
        q64, k64, v64, do64 = (t[n][0, h].to(torch.float64).numpy() for n in ("q", "k", "v", "do"))
        rows = pick_rows(r, w.nq, [np.searchsorted(mask_rows_all, gv[0])] if key == "c5" else gv)
        O, LSE, dQ = rows_reference(q64, k64, v64, do64, gv, rows, mask_rows_all[rows], scale)
        assert_close(f"O h={h}", f64(o[0, h, rows]), O, tol)
        assert_lse(f64(lse[0, h, rows]), LSE)
        assert_close(f"dQ h={h}", f64(dq[0, h, rows]), dQ, tol)
        n_cols = 8 if w.nk <= 8192 else (2 if w.family == "sliding_window" else 6)
        cols = pick_cols(r, w.nk, gv, mask_rows_all, max_rows, n=n_cols)
        assert cols.size > 0
        dK, dV = cols_reference(q64, k64, v64, do64, gv, cols, mask_rows_all, scale)
        assert_close(f"dK h={h}", f64(dk[0, h, cols]), dK, tol)
        assert_close(f"dV h={h}", f64(dv[0, h, cols]), dV, tol)
        print(f"  head {h}: {len(rows)} rows, {len(cols)} cols ok", flush=True)
