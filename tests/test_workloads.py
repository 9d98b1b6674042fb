"""Pins of the mask-family encodings: the four vectors, expanded by the oracle's ``dense_mask``,
must equal the brute-force family definition; the oracle's ``unmasked_count`` must equal the
dense count and each family's closed form."""

import numpy as np
import pytest

import oracle
from tests import families as fam
from workloads import configs, masks


def dense(v, nq=None):
    nq = len(v[0]) if nq is None else nq
    return oracle.dense_mask(*v, np.arange(nq))


def rng(*k):
    return np.random.default_rng(np.random.SeedSequence([99, *k]))


@pytest.mark.parametrize("n", [1, 2, 7, 33, 64])
def test_causal(n):
    v = masks.causal(n)
    assert (dense(v) == fam.causal(n)).all()
    assert oracle.unmasked_count(*v, n) == fam.unmasked_closed_form("causal", n)


@pytest.mark.parametrize("n,w", [(1, 1), (10, 1), (10, 3), (40, 7), (40, 40), (40, 100)])
def test_sliding_window(n, w):
    v = masks.sliding_window(n, w)
    assert (dense(v) == fam.sliding_window(n, w)).all()
    if w <= n:
        assert oracle.unmasked_count(*v, n) == fam.unmasked_closed_form("sliding_window", n, w=w)
    assert oracle.unmasked_count(*v, n) == int((~dense(v)).sum())


@pytest.mark.parametrize("seed", range(20))
def test_document(seed):
    r = rng(1, seed)
    n = int(r.integers(1, 80))
    k = int(r.integers(1, min(n, 9) + 1))
    L = masks.uniform_cut_lengths(r, n, k)
    assert L.sum() == n and L.min() >= 1 and len(L) == k
    v = masks.document(n, L)
    assert (dense(v) == fam.document(n, L)).all()
    assert oracle.unmasked_count(*v, n) == fam.unmasked_closed_form("document", n, lengths=L)


@pytest.mark.parametrize("seed", range(12))
def test_prefix_lm(seed):
    r = rng(2, seed)
    n = int(r.integers(2, 70))
    P = int(r.integers(0, n + 1))
    v = masks.prefix_lm(n, P)
    assert (dense(v) == fam.prefix_lm(n, P)).all()
    assert oracle.unmasked_count(*v, n) == fam.unmasked_closed_form("prefix_lm", n, prefix=P)


@pytest.mark.parametrize("seed", range(12))
def test_share_question(seed):
    r = rng(3, seed)
    n = int(r.integers(8, 90))
    q_len, ans = masks.draw_share_question(r, n, n_answers=4, q_lo=1, q_hi=n - 4)
    v = masks.share_question(n, q_len, ans)
    assert (dense(v) == fam.share_question(n, q_len, ans)).all()
    assert oracle.unmasked_count(*v, n) == fam.unmasked_closed_form(
        "share_question", n, q_len=q_len, answers=ans)


@pytest.mark.parametrize("seed", range(12))
def test_block_sparse(seed):
    r = rng(4, seed)
    block = int(r.integers(1, 9))
    n = int(r.integers(1, 70))
    a, z = masks.draw_block_sparse(r, n, block=block)
    v = masks.block_sparse(n, a, z, block=block)
    assert (dense(v) == fam.block_sparse(n, a, z, block=block)).all()
    assert oracle.unmasked_count(*v, n) == fam.unmasked_closed_form(
        "block_sparse", n, starts=a, ends=z, block=block)


@pytest.mark.parametrize("seed", range(10))
def test_unmasked_count_arbitrary_vectors(seed):
    """Interval arithmetic against the dense count on vectors with reversed, overlapping and
    out-of-range stretches."""
    r = rng(5, seed)
    nq, nk = int(r.integers(1, 40)), int(r.integers(1, 40))
    v = masks.random_vectors(r, nk, nq, spread=5)
    assert oracle.unmasked_count(*v, nq) == int((~oracle.dense_mask(*v, np.arange(nq))).sum())


def test_closed_form_counts_at_config_sizes():
    """Exact unmasked counts quoted for the n=8192 and n=131072 workloads."""
    assert oracle.unmasked_count(*masks.causal(8192), 8192) == 33_558_528
    assert oracle.unmasked_count(*masks.sliding_window(8192, 1024), 8192) == 7_864_832
    assert oracle.unmasked_count(*masks.sliding_window(131072, 4096), 131072) == 528_484_352


def test_lognormal_lengths():
    for s in range(5):
        L = masks.lognormal_lengths(rng(6, s), 32768, 40)
        assert L.sum() == 32768 and len(L) == 40 and L.min() >= 1 and L.max() <= 8192


def test_config_masks_are_deterministic_and_match_their_family():
    for key in ["c1", "c2c", "c2d", "c2e", "c2f"]:
        w = configs.WORKLOADS[key]
        v1 = configs.global_mask(w)
        v2 = configs.global_mask(w)
        for a, b in zip(v1, v2):
            assert (a == b).all()
        p = configs.family_params(w)
        n = w.nk
        fam_name = {"document_uniform": "document"}.get(w.family, w.family)
        if fam_name == "document":
            assert oracle.unmasked_count(*v1, n) == fam.unmasked_closed_form("document", n, **p)
        elif fam_name == "prefix_lm":
            assert 1024 <= p["prefix"] <= 4096
            assert oracle.unmasked_count(*v1, n) == fam.unmasked_closed_form(fam_name, n, **p)
        elif fam_name == "share_question":
            assert 512 <= p["q_len"] <= 2048 and len(p["answers"]) == 4
            assert oracle.unmasked_count(*v1, n) == fam.unmasked_closed_form(fam_name, n, **p)
        elif fam_name == "block_sparse":
            assert oracle.unmasked_count(*v1, n) == fam.unmasked_closed_form(fam_name, n, **p)


def test_c1_dense_matches_definition():
    w = configs.WORKLOADS["c1"]
    v = configs.global_mask(w)
    L = configs.family_params(w)["lengths"]
    assert len(L) == 3 and L.sum() == 256
    assert (dense(v) == fam.document(256, L)).all()


def test_tensor_streams_seeded_and_shaped():
    w = configs.WORKLOADS["c1"]
    t = configs.tensors(w)
    assert t["q"].shape == (1, 2, 256, 64) and str(t["q"].dtype) == "torch.float32"
    t2 = configs.tensors(w)
    assert all((t[k] == t2[k]).all() for k in t)
    assert not (t["q"] == t["k"]).all()
