"""Pins of the oracle's clip-shift-max localisation.

* Theorem 1 (FlashMask-3 explainer, clip-shift-max paragraph; abstract): the rank-local
  stretches reproduce the global ones at the owned rows, checked densely: the global dense mask
  restricted to the owned rows equals the local dense mask built from the localised vectors.
* An independent rank function: the localised mark equals the number of owned rows below it
  (numpy ``searchsorted`` over the sorted owned rows).
* Special cases: one chunk covering everything is the identity on in-range marks; the
  context-parallel rank of the 128K workload has hand-derived spot values.
"""

import numpy as np
import pytest

import oracle
from workloads import configs, masks


def rng(*k):
    return np.random.default_rng(np.random.SeedSequence([55, *k]))


def random_chunks(r, n):
    """1..4 sorted, disjoint, non-empty chunks inside [0, n]."""
    k = int(r.integers(1, min(4, (n + 1) // 2) + 1))
    pts = np.sort(r.choice(np.arange(n + 1), size=2 * k, replace=False))
    starts, ends = pts[0::2], pts[1::2]
    return starts, ends - starts


@pytest.mark.parametrize("seed", range(60))
def test_theorem1_dense(seed):
    r = rng(1, seed)
    n = int(r.integers(2, 60))
    o, L = random_chunks(r, n)
    v = masks.random_vectors(r, n, n, spread=int(r.integers(0, 4)))
    lv = oracle.localize(*v, o, L, n)
    n_local = lv[4]
    owned = np.concatenate([np.arange(a, a + b) for a, b in zip(o, L)])
    assert n_local == len(owned)
    glob = oracle.dense_mask(*v, owned)
    loc = oracle.dense_mask(*lv[:4], np.arange(n_local))
    assert (glob == loc).all()
    for x in lv[:4]:
        assert x.dtype == np.int32 and x.min() >= 0 and x.max() <= n_local


@pytest.mark.parametrize("seed", range(30))
def test_rank_function(seed):
    r = rng(2, seed)
    n = int(r.integers(2, 200))
    o, L = random_chunks(r, n)
    owned = np.concatenate([np.arange(a, a + b) for a, b in zip(o, L)])
    x = r.integers(-20, n + 20, size=300)
    out = oracle.localize(x, x, x, x, o, L, n)
    assert (out[0] == np.searchsorted(owned, x, side="left")).all()


def test_single_chunk_identity():
    x = np.arange(-5, 70)
    out = oracle.localize(x, x, x, x, [0], [64], 64)
    assert (out[0] == np.clip(x, 0, 64)).all() and out[4] == 64


def test_cp_rank_spot_values():
    """Rank 5 of 16 with dual-chunk assignment over 32 chunks of 4096: it owns global rows
    [20480, 24576) and [106496, 110592), local rows [0, 4096) and [4096, 8192).  A mark counts
    the owned rows below it: 22000 -> 22000 - 20480 = 1520; anything in the gap -> 4096;
    110000 -> 4096 + (110000 - 106496) = 7600; anything at or past 110592 -> 8192."""
    x = np.array([0, 20480, 22000, 24576, 50000, 106496, 110000, 110592, 131072], dtype=np.int32)
    out = oracle.localize(x, x, x, x, configs.C5_CHUNK_START, configs.C5_CHUNK_LEN, 131072)
    assert out[0].tolist() == [0, 0, 1520, 4096, 4096, 4096, 7600, 8192, 8192]
    assert out[4] == 8192


def test_cp_rank_theorem1_on_document_mask_rows():
    """Theorem 1 on the 128K context-parallel workload's own document mask, sampled rows."""
    w = configs.WORKLOADS["c5"]
    v = configs.global_mask(w)
    lv = oracle.localize(*v, configs.C5_CHUNK_START, configs.C5_CHUNK_LEN, 131072)
    owned = configs.owned_rows(w)
    pick = rng(3).choice(len(owned), size=24, replace=False)
    glob = oracle.dense_mask(*v, owned[pick])
    loc = oracle.dense_mask(*lv[:4], pick)
    assert (glob == loc).all()


@pytest.mark.parametrize("o,L", [([4, 0], [2, 2]),          # unsorted
                                 ([0, 1], [2, 2]),          # overlapping
                                 ([0], [0]),                # empty chunk
                                 ([60], [8]),               # past the end
                                 ([-1], [2]),               # negative offset
                                 ([], [])])
def test_invalid_chunk_tables(o, L):
    x = np.arange(4)
    with pytest.raises(ValueError):
        oracle.localize(x, x, x, x, o, L, 64)


def test_two_sided_clamp_reading_breaks_theorem1():
    """The literal 'clamp to [o, o+L], shift, max' reading disagrees with the rank function when
    a rank owns two chunks (a later chunk above the mark contributes its prefix): the reading
    taken by the oracle (clip only the upper end) is the one Theorem 1 needs."""
    o, L = np.array([2, 10]), np.array([3, 4])
    x = np.array([0, 1, 2, 3, 5, 7, 10, 12, 14, 20])
    P = np.array([0, 3])
    two_sided = np.max([np.clip(x, ok, ok + Lk) - ok + Pk for ok, Lk, Pk in zip(o, L, P)], axis=0)
    owned = np.concatenate([np.arange(a, a + b) for a, b in zip(o, L)])
    rank = np.searchsorted(owned, x)
    assert (two_sided != rank).any()
    assert (oracle.localize(x, x, x, x, o, L, 20)[0] == rank).all()
