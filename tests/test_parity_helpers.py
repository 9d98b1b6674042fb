"""CPU checks of the GPU tests' oracle drivers (no GPU): the whole-head driver, which runs the
oracle's row functions on exact sub-problems (only the keys some row of a block can see), equals
the oracle's plain dense drivers, including fully masked rows, several row blocks, a ragged last
block and context-parallel row numbering."""

import numpy as np
import pytest

import oracle
from tests.parity import whole_head_reference
from workloads import masks


def data(r, nq, nk, d=16):
    return [r.standard_normal((n, d)) for n in (nq, nk, nk, nq)]


@pytest.mark.parametrize("kind", ["document", "swa", "random", "padrows"])
def test_whole_head_equals_dense_oracle(kind):
    r = np.random.default_rng(np.random.SeedSequence([31, len(kind)]))
    n = 300
    if kind == "document":
        vec = masks.document(n, masks.uniform_cut_lengths(r, n, 7))
    elif kind == "swa":
        vec = masks.sliding_window(n, 37)
    elif kind == "random":
        vec = masks.random_vectors(r, n, n, spread=10)
    else:  # the last 50 rows fully masked
        vec = (np.full(n, n - 50, np.int32), np.full(n, n, np.int32), np.zeros(n, np.int32),
               np.arange(n, dtype=np.int32))
    q, k, v, do = data(r, n, n)
    scale = 0.25
    O, LSE, dQ, dK, dV = whole_head_reference(q, k, v, do, vec, np.arange(n), scale,
                                              row_block=64, workers=3)
    O2, LSE2 = oracle.attention_fwd(q[None, None], k[None, None], v[None, None], vec, scale)
    dQ2, dK2, dV2 = oracle.attention_bwd(q[None, None], k[None, None], v[None, None],
                                         do[None, None], vec, scale)
    assert np.array_equal(np.isneginf(LSE), np.isneginf(LSE2[0, 0]))
    fin = np.isfinite(LSE)
    np.testing.assert_allclose(LSE[fin], LSE2[0, 0][fin], rtol=0, atol=1e-12)
    for a, b in ((O, O2), (dQ, dQ2), (dK, dK2), (dV, dV2)):
        np.testing.assert_allclose(a, b[0, 0], rtol=0, atol=1e-11)


def test_whole_head_with_global_row_numbers():
    """Local rows that are a subset of a global problem's rows (a context-parallel share): the
    driver with global row numbers equals the dense oracle on the global mask at those rows."""
    r = np.random.default_rng(5)
    n = 256
    vec = masks.document(n, masks.uniform_cut_lengths(r, n, 5))
    rows = np.concatenate([np.arange(32, 64), np.arange(192, 224)])
    q, k, v, do = data(r, len(rows), n)
    O, LSE, dQ, dK, dV = whole_head_reference(q, k, v, do, vec, rows, 0.3, row_block=16,
                                              workers=2)
    O2, LSE2 = oracle.attention_fwd(q[None, None], k[None, None], v[None, None], vec, 0.3,
                                    rows=rows)
    dQ2, dK2, dV2 = oracle.attention_bwd(q[None, None], k[None, None], v[None, None],
                                         do[None, None], vec, 0.3, rows=rows)
    for a, b in ((O, O2), (dQ, dQ2), (dK, dK2), (dV, dV2)):
        np.testing.assert_allclose(a, b[0, 0], rtol=0, atol=1e-11)
