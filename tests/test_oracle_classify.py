"""Pins of the oracle's tile classification: a brute-force scan of the dense mask over every
tile decides which tiles are truly fully masked / unmasked.  The oracle's classes must be sound
on arbitrary vectors and exact on the structured families at the kernel tile shapes."""

import numpy as np
import pytest

import oracle
from tests import families as fam
from workloads import masks


def rng(*k):
    return np.random.default_rng(np.random.SeedSequence([77, *k]))


def brute_tiles(M, BM, BN):
    """For every tile: 0 if every entry masked, 2 if none, 1 otherwise (tail tiles are clipped)."""
    nq, nk = M.shape
    n_qb, n_kb = -(-nq // BM), -(-nk // BN)
    out = np.empty((n_qb, n_kb), dtype=np.uint8)
    for qb in range(n_qb):
        for kb in range(n_kb):
            t = M[qb * BM:(qb + 1) * BM, kb * BN:(kb + 1) * BN]
            out[qb, kb] = 0 if t.all() else (2 if not t.any() else 1)
    return out


def check_lists(c):
    cls = c["cls"]
    n_qb, n_kb = cls.shape
    for qb in range(n_qb):
        exp = [kb * 2 + int(cls[qb, kb] == 1) for kb in range(n_kb) if cls[qb, kb]]
        assert c["qlist"][qb] == exp and c["qcnt"][qb] == len(exp)
    for kb in range(n_kb):
        exp = [qb * 2 + int(cls[qb, kb] == 1) for qb in range(n_qb) if cls[qb, kb]]
        assert c["klist"][kb] == exp and c["kcnt"][kb] == len(exp)


def test_block_minmax_against_numpy_reduce():
    v = rng(0).integers(-1000, 1000, size=1001)
    for BN in (1, 2, 3, 64, 1000, 1001, 2000):
        mins, maxs = oracle.block_minmax(v, BN)
        n_kb = -(-len(v) // BN)
        assert len(mins) == n_kb
        pad = np.full(n_kb * BN, np.iinfo(np.int64).max)
        pad[:len(v)] = v
        assert (mins == pad.reshape(n_kb, BN).min(1)).all()
        pad[len(v):] = np.iinfo(np.int64).min
        assert (maxs == pad.reshape(n_kb, BN).max(1)).all()


@pytest.mark.parametrize("seed", range(40))
def test_sound_on_arbitrary_vectors(seed):
    r = rng(1, seed)
    nq, nk = int(r.integers(1, 48)), int(r.integers(1, 48))
    BM, BN = int(r.integers(1, 17)), int(r.integers(1, 17))
    v = masks.random_vectors(r, nk, nq, spread=int(r.integers(0, 6)))
    M = oracle.dense_mask(*v, np.arange(nq))
    c = oracle.classify(*v, nq, BM, BN)
    truth = brute_tiles(M, BM, BN)
    # soundness: a skipped tile is truly all-masked; an untested tile is truly unmasked
    assert ((c["cls"] == 0) <= (truth == 0)).all()
    assert ((c["cls"] == 2) <= (truth == 2)).all()
    check_lists(c)


def _family_vectors(r, n):
    w = int(r.integers(1, n + 1))
    L = masks.uniform_cut_lengths(r, n, int(r.integers(1, min(n, 6) + 1)))
    P = int(r.integers(0, n + 1))
    q_len, ans = masks.draw_share_question(r, n, 4, 1, n - 4)
    a, z = masks.draw_block_sparse(r, n, block=16)
    return {
        "causal": (masks.causal(n), fam.causal(n)),
        "swa": (masks.sliding_window(n, w), fam.sliding_window(n, w)),
        "document": (masks.document(n, L), fam.document(n, L)),
        "prefix_lm": (masks.prefix_lm(n, P), fam.prefix_lm(n, P)),
        "share_question": (masks.share_question(n, q_len, ans), fam.share_question(n, q_len, ans)),
        "block_sparse": (masks.block_sparse(n, a, z, 16), fam.block_sparse(n, a, z, 16)),
    }


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("BM,BN", [(4, 4), (8, 4), (4, 8), (16, 16), (8, 16), (16, 8), (5, 4)])
def test_exact_on_families(seed, BM, BN):
    """On the structured families the rule is exact (no conservative tile) whenever the key
    block width divides the block-sparse block (16 here)."""
    r = rng(2, seed, BM, BN)
    n = int(r.integers(8, 70))
    for name, (v, brute) in _family_vectors(r, n).items():
        M = oracle.dense_mask(*v, np.arange(n))
        assert (M == brute).all(), name
        c = oracle.classify(*v, n, BM, BN)
        truth = brute_tiles(brute, BM, BN)
        assert (c["cls"] == truth).all(), name
        check_lists(c)


def test_tile_counts_at_kernel_shapes_causal():
    """Causal n=1024, 128x64 tiles: query block qb (rows 128qb..) sees key blocks 0..2qb+1, of
    which the two on the diagonal are partial."""
    c = oracle.classify(*masks.causal(1024), 1024, 128, 64)
    for qb in range(8):
        assert c["qcnt"][qb] == 2 * qb + 2
        partial = [e & 1 for e in c["qlist"][qb]]
        assert partial == [0] * (2 * qb) + [1, 1]
