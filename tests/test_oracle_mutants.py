"""Planted mistakes: each mutant below is a plausible slip in the oracle (a closed interval, a
dropped stretch, a missing scale, a dropped term, a wrong operand, an unsound bound, an
off-by-one block, the two-sided clamp, a prune list that drops partly masked chunks).  Each must be caught by at least one of the pins in the
oracle's tests, which shows the pins constrain the oracle rather than restate it.  The mistakes
are planted in the oracle only, on the CPU."""

import numpy as np
import pytest

import oracle
import oracle.flashmask_oracle as fo
from tests import test_oracle_attention as ta
from tests import test_oracle_classify as tc
from tests import test_oracle_localize as tl
from tests import test_oracle_prune as tp
from tests import test_workloads as tw

_orig = {n: getattr(fo, n) for n in ("dense_mask", "fwd_rows", "bwd_rows", "block_minmax",
                                     "classify", "localize", "prune_chunks")}


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(fo, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def closed_interval_mask(LTS, LTE, UTS, UTE, rows):
    i = np.asarray(rows, dtype=np.int64)[:, None]
    a, b, c, d = (np.asarray(x, dtype=np.int64)[None, :] for x in (LTS, LTE, UTS, UTE))
    return ((a <= i) & (i <= b)) | ((c <= i) & (i <= d))


def lt_only_mask(LTS, LTE, UTS, UTE, rows):
    i = np.asarray(rows, dtype=np.int64)[:, None]
    a, b = (np.asarray(x, dtype=np.int64)[None, :] for x in (LTS, LTE))
    return (a <= i) & (i < b)


def fwd_no_scale(q, K, V, masked, scale):
    return _orig["fwd_rows"](q, K, V, masked, 1.0)


def bwd_dk_no_scale(q, K, V, dO, masked, scale, cols=None):
    dq, dk, dv = _orig["bwd_rows"](q, K, V, dO, masked, scale, cols)
    return dq, dk / scale, dv


def bwd_no_D(q, K, V, dO, masked, scale, cols=None):
    q, K, V, dO = (np.asarray(x, np.float64) for x in (q, K, V, dO))
    O, LSE = _orig["fwd_rows"](q, K, V, masked, scale)
    S = scale * q @ K.T
    live = np.isfinite(LSE)
    P = np.zeros_like(S)
    P[live] = np.exp(np.where(masked[live], -np.inf, S[live]) - LSE[live][:, None])
    dS = P * (dO @ V.T)                       # the "- D" term dropped
    dk = scale * dS.T @ q
    dv = P.T @ dO
    if cols is not None:
        dk, dv = dk[cols], dv[cols]
    return scale * dS @ K, dk, dv


def bwd_dq_wrong_operand(q, K, V, dO, masked, scale, cols=None):
    dq, dk, dv = _orig["bwd_rows"](q, K, V, dO, masked, scale, cols)
    q, K, V, dO = (np.asarray(x, np.float64) for x in (q, K, V, dO))
    # rebuild dq with V in place of K
    O, LSE = _orig["fwd_rows"](q, K, V, masked, scale)
    S = scale * q @ K.T
    live = np.isfinite(LSE)
    P = np.zeros_like(S)
    P[live] = np.exp(np.where(masked[live], -np.inf, S[live]) - LSE[live][:, None])
    dS = P * (dO @ V.T - (dO * O).sum(1)[:, None])
    return scale * dS @ V, dk, dv


def minmax_off_by_one(vec, BN):
    v = np.asarray(vec, dtype=np.int64)
    n_kb = -(-len(v) // BN)
    mins = np.array([v[b * BN:min((b + 1) * BN + 1, len(v))].min() for b in range(n_kb)])
    maxs = np.array([v[b * BN:min((b + 1) * BN + 1, len(v))].max() for b in range(n_kb)])
    return mins, maxs


def classify_unsound(LTS, LTE, UTS, UTE, nq, BM, BN):
    # LT "full" tested against the block maximum of LTE instead of its minimum
    out = _orig["classify"](LTS, LTE, UTS, UTE, nq, BM, BN)
    lts_lo, lts_hi = fo.block_minmax(LTS, BN)
    lte_lo, lte_hi = fo.block_minmax(LTE, BN)
    n_qb = -(-nq // BM)
    r0 = (np.arange(n_qb) * BM)[:, None]
    r1 = np.minimum(r0 + BM, nq)
    bad_full = (lts_hi[None, :] <= r0) & (lte_hi[None, :] >= r1)
    out["cls"] = np.where(bad_full, 0, out["cls"]).astype(np.uint8)
    return out


def localize_two_sided(LTS, LTE, UTS, UTE, chunk_start, chunk_len, nq_global):
    o, L = fo.localize_chunks_check(chunk_start, chunk_len, nq_global)
    P = np.concatenate([[0], np.cumsum(L)[:-1]])

    def ell(x):
        x = np.asarray(x, dtype=np.int64)
        return np.max([np.clip(x, ok, ok + Lk) - ok + Pk for ok, Lk, Pk in zip(o, L, P)],
                      axis=0).astype(np.int32)
    return ell(LTS), ell(LTE), ell(UTS), ell(UTE), int(L.sum())


def prune_counts_unmasked_only(LTS, LTE, UTS, UTE, n_local, BM, chunk):
    # counts only tiles with no masked entry, so chunks seen through partial tiles are pruned
    cls = fo.classify(LTS, LTE, UTS, UTE, n_local, BM, chunk)["cls"]
    return (cls == 2).sum(axis=0).astype(np.int64)


def _doc_seed0():
    tw.test_document(3)
    tw.test_sliding_window(40, 7)


def _sdpa():
    for s in range(3):
        ta.test_forward_matches_sdpa_on_families(s)


def _bwd_pins():
    for s in range(2):
        ta.test_backward_finite_differences(s)


MUTANTS = [
    ("dense_mask", closed_interval_mask, _doc_seed0),
    ("dense_mask", lt_only_mask, _doc_seed0),
    ("fwd_rows", fwd_no_scale, _sdpa),
    ("bwd_rows", bwd_dk_no_scale, _bwd_pins),
    ("bwd_rows", bwd_no_D, _bwd_pins),
    ("bwd_rows", bwd_dq_wrong_operand, _bwd_pins),
    ("block_minmax", minmax_off_by_one, tc.test_block_minmax_against_numpy_reduce),
    ("classify", classify_unsound, lambda: [tc.test_sound_on_arbitrary_vectors(s) for s in range(40)]),
    ("localize", localize_two_sided, lambda: [tl.test_theorem1_dense(s) for s in range(60)]),
    ("prune_chunks", prune_counts_unmasked_only,
     lambda: [tp.test_pruned_chunks_are_fully_masked(s) for s in range(40)]),
]


@pytest.mark.parametrize("name,mutant,pins", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pins):
    pins()  # the real oracle passes
    _patch(monkeypatch, name, mutant)
    with pytest.raises(AssertionError):
        pins()
