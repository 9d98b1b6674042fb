"""Helpers shared by the GPU parity tests: tolerances, oracle values for sampled rows and key
columns, and comparisons.

Sampled oracle values call the oracle's own row functions on an exact sub-problem: for a set of
query rows only the keys that are unmasked for at least one of those rows are passed (every other
key is masked for all of them, so its probability is exactly zero and it adds nothing to any sum);
for a set of key columns only the rows with an unmasked entry in those columns contribute.
"""

from __future__ import annotations

import os
import threading
from concurrent.futures import FIRST_COMPLETED, ThreadPoolExecutor, wait

import numpy as np
import torch

import oracle

# Tolerances fixed by the target: max-abs error against the float64 oracle.
TOL = {"bf16": 2e-2, "fp32": 1e-4}
TOL_LSE = 1e-3


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def dev_i32(x, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


def rows_reference(q, k, v, do, vectors, rows, mask_rows, scale):
    """O, LSE and dQ of the given rows of one (batch, head); arrays are float64 numpy.

    q, do: [nq, d]; k, v: [nk, d]; rows: indices into q; mask_rows: the mask-row number of each
    selected row (global numbering for a context-parallel share)."""
    M = oracle.dense_mask(*vectors, mask_rows)
    keys = np.flatnonzero(~M.all(axis=0))
    if keys.size == 0:
        keys = np.array([0])
    Ms = M[:, keys]
    O, LSE = oracle.fwd_rows(q[rows], k[keys], v[keys], Ms, scale)
    dq = None
    if do is not None:
        dq, _, _ = oracle.bwd_rows(q[rows], k[keys], v[keys], do[rows], Ms, scale,
                                   cols=np.zeros(0, dtype=np.int64))
    return O, LSE, dq


def cols_reference(q, k, v, do, vectors, cols, mask_rows_all, scale):
    """dK and dV of the given key columns of one (batch, head)."""
    vc = [np.asarray(x)[cols] for x in vectors]
    Mc = oracle.dense_mask(*vc, mask_rows_all)
    R = np.flatnonzero(~Mc.all(axis=1))
    d = k.shape[1]
    if R.size == 0:
        return np.zeros((len(cols), d)), np.zeros((len(cols), v.shape[1]))
    M = oracle.dense_mask(*vectors, mask_rows_all[R])
    keys = np.union1d(np.flatnonzero(~M.all(axis=0)), cols)
    pos = np.searchsorted(keys, cols)
    _, dk, dv = oracle.bwd_rows(q[R], k[keys], v[keys], do[R], M[:, keys], scale, cols=pos)
    return dk, dv


def oracle_workers():
    """Worker threads for the whole-head oracle: the cores this process may use, at most 16 (the
    host share one GPU typically gets)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def whole_head_reference(q, k, v, do, vectors, mask_rows, scale, row_block=128, workers=None):
    """O, LSE, dQ (every query row) and dK, dV (every key column) of one (batch, head), in float64.

    The oracle's own row functions run on exact sub-problems: for each block of ``row_block``
    consecutive query rows only the keys that are unmasked for at least one of those rows take
    part (every other key is masked for all of them, so it has probability exactly zero and adds
    nothing to any sum).  Each block's dQ is complete; its dK / dV contributions at those keys
    are summed over the blocks.  Blocks run on a thread pool (numpy and BLAS release the GIL;
    BLAS at one thread per worker), at most 2 x workers blocks in flight so memory stays
    bounded.  q, do: [nq, d]; k, v: [nk, d] (float64 arrays); mask_rows: mask-row number of each
    query row (global numbering for a context-parallel share)."""
    from threadpoolctl import threadpool_limits

    nq, d = q.shape
    nk = k.shape[0]
    mask_rows = np.asarray(mask_rows)
    O = np.zeros((nq, v.shape[1]))
    LSE = np.full(nq, -np.inf)
    dQ = np.zeros((nq, d))
    dK = np.zeros((nk, d))
    dV = np.zeros((nk, v.shape[1]))
    lock = threading.Lock()

    def block(r0):
        r1 = min(nq, r0 + row_block)
        M = oracle.dense_mask(*vectors, mask_rows[r0:r1])
        keys = np.flatnonzero(~M.all(axis=0))
        if keys.size == 0:
            return  # every row fully masked: O = 0, LSE = -inf, no gradient anywhere
        Ms = M[:, keys]
        o, lse = oracle.fwd_rows(q[r0:r1], k[keys], v[keys], Ms, scale)
        dq, dk, dv = oracle.bwd_rows(q[r0:r1], k[keys], v[keys], do[r0:r1], Ms, scale)
        O[r0:r1], LSE[r0:r1], dQ[r0:r1] = o, lse, dq
        with lock:
            dK[keys] += dk
            dV[keys] += dv

    workers = workers or oracle_workers()
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers) as ex:
        pending = set()
        for r0 in range(0, nq, row_block):
            if len(pending) >= 2 * workers:
                done, pending = wait(pending, return_when=FIRST_COMPLETED)
                for f in done:
                    f.result()
            pending.add(ex.submit(block, r0))
        for f in pending:
            f.result()
    return O, LSE, dQ, dK, dV


def column_cost(vectors, col, mask_rows_all):
    """Rough work of cols_reference for one column: rows attending it x their key span."""
    vc = [np.asarray(x)[[col]] for x in vectors]
    Mc = oracle.dense_mask(*vc, mask_rows_all)
    return int((~Mc).sum())


def assert_close(name, got, want, tol):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert not np.isnan(got).any(), f"{name}: NaN in GPU output"
    err = np.abs(got - want).max() if got.size else 0.0
    if os.environ.get("FM_PARITY_REPORT"):
        print(f"parity {name}: max-abs error {err:.3e} (tolerance {tol:.1e})", flush=True)
    assert err <= tol, f"{name}: max-abs error {err:.3e} > {tol:.1e}"
    return err


def assert_lse(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert not np.isnan(got).any(), "LSE: NaN"
    ninf_g, ninf_w = np.isneginf(got), np.isneginf(want)
    assert np.array_equal(ninf_g, ninf_w), "LSE: -inf rows differ"
    live = ~ninf_w
    err = np.abs(got[live] - want[live]).max() if live.any() else 0.0
    assert err <= TOL_LSE, f"LSE: max-abs error {err:.3e} > {TOL_LSE:.0e}"
    return err
