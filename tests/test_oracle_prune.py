"""Pins of the oracle's key/value chunk prune list (the decision half of mask-driven
communication pruning; FlashMask-3 explainer, across-ranks paragraph).

* Soundness on arbitrary vectors: a chunk the rule prunes is fully masked for every local row
  (dense brute force over the rank's rows and the chunk's keys).
* Exactness on the causal, document and sliding-window families for context-parallel shares
  whose query blocks are the rank's own chunks: the count equals the number of owned row chunks
  that see at least one key of the chunk (dense brute force on the *global* mask at the owned
  rows, so localisation is checked along the way).
* Closed form: under a causal mask, a rank owning row chunks {r, 2R-1-r} of 2R equal chunks
  needs key chunk c from the row chunks at or after c.
"""

import numpy as np
import pytest

import oracle
from workloads import masks


def rng(*k):
    return np.random.default_rng(np.random.SeedSequence([71, *k]))


def zigzag(R, r, L):
    """Row chunks r and 2R-1-r of length L (the dual-chunk assignment)."""
    return np.array([r * L, (2 * R - 1 - r) * L]), np.array([L, L])


@pytest.mark.parametrize("seed", range(40))
def test_pruned_chunks_are_fully_masked(seed):
    r = rng(1, seed)
    n_local = int(r.integers(1, 50))
    nk = int(r.integers(1, 80))
    BM = int(r.integers(1, 20))
    chunk = int(r.integers(1, 20))
    v = masks.random_vectors(r, nk, n_local, spread=int(r.integers(0, 3)))
    live = oracle.prune_chunks(*v, n_local, BM, chunk)
    dense = oracle.dense_mask(*v, np.arange(n_local))
    for c in range(len(live)):
        block = dense[:, c * chunk:(c + 1) * chunk]
        if live[c] == 0:
            assert block.all()
        # the count never exceeds the number of query blocks
        assert 0 <= live[c] <= -(-n_local // BM)


def _family(name, r, n):
    if name == "causal":
        return masks.causal(n)
    if name == "document":
        return masks.document(n, masks.uniform_cut_lengths(r, n, int(r.integers(1, min(8, n) + 1))))
    return masks.sliding_window(n, int(r.integers(1, n + 1)))


@pytest.mark.parametrize("name", ["causal", "document", "swa"])
@pytest.mark.parametrize("seed", range(12))
def test_exact_on_families_for_cp_shares(name, seed):
    r = rng(2, seed, ["causal", "document", "swa"].index(name))
    R = int(r.integers(1, 5))
    L = int(r.integers(1, 9))
    n = 2 * R * L
    rank = int(r.integers(0, R))
    chunk = int(r.integers(1, 2 * L + 1))
    v = _family(name, r, n)
    o, lens = zigzag(R, rank, L)
    if R == 1:
        o, lens = np.array([0]), np.array([n])
    lv = oracle.localize(*v, o, lens, n)
    BM = int(lens[0])
    live = oracle.prune_chunks(*lv[:4], lv[4], BM, chunk)
    want = []
    for c in range(-(-n // chunk)):
        k = 0
        for a, b in zip(o, lens):
            rows = np.arange(a, a + b)
            if not oracle.dense_mask(*v, rows)[:, c * chunk:(c + 1) * chunk].all():
                k += 1
        want.append(k)
    assert live.tolist() == want


def test_causal_closed_form():
    R, L = 4, 16
    n = 2 * R * L
    v = masks.causal(n)
    for rank in range(R):
        o, lens = zigzag(R, rank, L)
        lv = oracle.localize(*v, o, lens, n)
        live = oracle.prune_chunks(*lv[:4], lv[4], L, L)
        owned = [rank, 2 * R - 1 - rank]
        assert live.tolist() == [sum(1 for q in owned if q >= c) for c in range(2 * R)]
