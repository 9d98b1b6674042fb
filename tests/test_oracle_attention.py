"""Pins of the oracle's attention forward and backward.

Forward: closed form at Q = 0; torch SDPA (float64, CPU) with the brute-force family masks;
torch logsumexp for LSE; the bound m <= LSE <= m + ln(count); fully masked rows.
Backward: central finite differences of L = sum(O * dO) in float64; torch autograd through SDPA
in float64; the exact identities sum_j dK_j = 0 and sum_j dV_j = sum over live rows of dO_i.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tests import families as fam
from workloads import masks


def rng(*k):
    return np.random.default_rng(np.random.SeedSequence([33, *k]))


def rand(r, *shape):
    return r.standard_normal(shape)


def family_cases(r, n):
    L = masks.uniform_cut_lengths(r, n, int(r.integers(1, 5)))
    P = int(r.integers(1, n))
    q_len, ans = masks.draw_share_question(r, n, 3, 1, n - 3)
    a, z = masks.draw_block_sparse(r, n, block=4)
    w = int(r.integers(1, n))
    return [
        (masks.no_mask(n), np.zeros((n, n), bool)),
        (masks.causal(n), fam.causal(n)),
        (masks.sliding_window(n, w), fam.sliding_window(n, w)),
        (masks.document(n, L), fam.document(n, L)),
        (masks.prefix_lm(n, P), fam.prefix_lm(n, P)),
        (masks.share_question(n, q_len, ans), fam.share_question(n, q_len, ans)),
        (masks.block_sparse(n, a, z, 4), fam.block_sparse(n, a, z, 4)),
    ]


def sdpa(q, k, v, brute_masked, scale):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    return F.scaled_dot_product_attention(t(q)[None], t(k)[None], t(v)[None],
                                          attn_mask=t(~brute_masked)[None], scale=scale)[0].numpy()


@pytest.mark.parametrize("seed", range(6))
def test_forward_matches_sdpa_on_families(seed):
    r = rng(1, seed)
    n, d = int(r.integers(5, 40)), int(r.integers(1, 9))
    scale = float(r.uniform(0.2, 1.5))
    for v, brute in family_cases(r, n):
        q, k, vv = rand(r, n, d), rand(r, n, d), rand(r, n, d)
        O, LSE = oracle.fwd_rows(q, k, vv, oracle.dense_mask(*v, np.arange(n)), scale)
        ref = sdpa(q, k, vv, brute, scale)
        live = ~brute.all(1)
        assert np.allclose(O[live], ref[live], atol=1e-12, rtol=1e-10)
        S = torch.from_numpy(scale * q @ k.T).masked_fill(torch.from_numpy(brute), -math.inf)
        lse_ref = torch.logsumexp(S, dim=1).numpy()
        assert np.allclose(LSE[live], lse_ref[live], atol=1e-12, rtol=1e-12)


def test_forward_closed_form_zero_queries():
    """Q = 0: every live score is 0, so O_i is the mean of the unmasked V_j and LSE_i = ln(count)."""
    r = rng(2)
    nq, nk, d = 23, 31, 5
    v = masks.random_vectors(r, nk, nq, spread=3)
    M = oracle.dense_mask(*v, np.arange(nq))
    V = rand(r, nk, d)
    O, LSE = oracle.fwd_rows(np.zeros((nq, d)), rand(r, nk, d), V, M, 0.7)
    for i in range(nq):
        keep = ~M[i]
        if keep.any():
            assert np.allclose(O[i], V[keep].mean(0), atol=1e-13)
            assert abs(LSE[i] - math.log(keep.sum())) < 1e-13
        else:
            assert (O[i] == 0).all() and LSE[i] == -math.inf


def test_forward_lse_bounds():
    r = rng(3)
    nq, nk, d = 40, 37, 8
    v = masks.random_vectors(r, nk, nq, spread=2)
    M = oracle.dense_mask(*v, np.arange(nq))
    q, k = rand(r, nq, d), rand(r, nk, d)
    _, LSE = oracle.fwd_rows(q, k, rand(r, nk, d), M, 0.35)
    S = 0.35 * q @ k.T
    for i in range(nq):
        keep = ~M[i]
        if keep.any():
            m = S[i][keep].max()
            assert m - 1e-12 <= LSE[i] <= m + math.log(keep.sum()) + 1e-12


def test_fully_masked_rows_forward_and_backward():
    """Causal plus the last ``pad`` rows closed for every key: those rows get O = 0,
    LSE = -inf, dQ = 0, and contribute nothing to dK and dV."""
    r = rng(4)
    n, d, pad = 24, 6, 5
    LTS, LTE, UTS, UTE = masks.causal(n)
    LTS = np.full(n, n - pad, np.int32)
    LTE = np.full(n, n, np.int32)
    v = (LTS, LTE, UTS, UTE)
    q, k, vv, do = (rand(r, 1, 1, n, d) for _ in range(4))
    O, LSE = oracle.attention_fwd(q, k, vv, v, 0.5)
    assert (O[0, 0, n - pad:] == 0).all() and np.isneginf(LSE[0, 0, n - pad:]).all()
    assert np.isfinite(LSE[0, 0, :n - pad]).all()
    dQ, dK, dV = oracle.attention_bwd(q, k, vv, do, v, 0.5)
    assert (dQ[0, 0, n - pad:] == 0).all()
    do2 = do.copy()
    do2[0, 0, n - pad:] = rand(r, pad, d)
    dQ2, dK2, dV2 = oracle.attention_bwd(q, k, vv, do2, v, 0.5)
    assert np.array_equal(dK, dK2) and np.array_equal(dV, dV2)


def loss(q, k, v, do, M, scale):
    O, _ = oracle.fwd_rows(q, k, v, M, scale)
    return float((O * do).sum())


@pytest.mark.parametrize("seed", range(4))
def test_backward_finite_differences(seed):
    r = rng(5, seed)
    nq, nk, d = 9, 11, 4
    scale = 0.6
    v = masks.random_vectors(r, nk, nq, spread=2)
    M = oracle.dense_mask(*v, np.arange(nq))
    q, k, vv, do = rand(r, nq, d), rand(r, nk, d), rand(r, nk, d), rand(r, nq, d)
    dq, dk, dv = oracle.bwd_rows(q, k, vv, do, M, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", vv, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": vv}
            args[name] = xp
            fp = loss(args["q"], args["k"], args["v"], do, M, scale)
            args[name] = xm
            fm = loss(args["q"], args["k"], args["v"], do, M, scale)
            num[idx] = (fp - fm) / (2 * h)
        assert np.allclose(g, num, atol=1e-7, rtol=1e-6), name


@pytest.mark.parametrize("seed", range(3))
def test_backward_matches_torch_autograd_on_families(seed):
    r = rng(6, seed)
    n, d = int(r.integers(6, 30)), int(r.integers(2, 7))
    scale = 0.8
    for v, brute in family_cases(r, n):
        if brute.all(1).any():
            continue  # SDPA returns NaN on fully masked rows; covered separately
        q, k, vv, do = (rand(r, n, d) for _ in range(4))
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, vv))
        out = F.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                             attn_mask=torch.from_numpy(~brute)[None],
                                             scale=scale)[0]
        out.backward(torch.from_numpy(do))
        dq, dk, dv = oracle.bwd_rows(q, k, vv, do, oracle.dense_mask(*v, np.arange(n)), scale)
        assert np.allclose(dq, tq.grad.numpy(), atol=1e-11)
        assert np.allclose(dk, tk.grad.numpy(), atol=1e-11)
        assert np.allclose(dv, tv.grad.numpy(), atol=1e-11)


def test_backward_identities_and_row_blocking():
    """sum_j dK_j = 0 and sum_j dV_j = sum_{live i} dO_i; the row-blocked driver equals one
    block; column-restricted contributions equal the full ones."""
    r = rng(7)
    B, H, nq, nk, d = 1, 2, 37, 29, 5
    v = masks.random_vectors(r, nk, nq, spread=1)
    Q, K, V, dO = rand(r, B, H, nq, d), rand(r, B, H, nk, d), rand(r, B, H, nk, d), rand(r, B, H, nq, d)
    dQ, dK, dV = oracle.attention_bwd(Q, K, V, dO, v, 0.45, row_block=7)
    dQ1, dK1, dV1 = oracle.attention_bwd(Q, K, V, dO, v, 0.45, row_block=1000, workers=2)
    assert np.allclose(dQ, dQ1, atol=1e-13) and np.allclose(dK, dK1, atol=1e-13)
    assert np.allclose(dV, dV1, atol=1e-13)
    _, LSE = oracle.attention_fwd(Q, K, V, v, 0.45)
    for h in range(H):
        assert np.allclose(dK[0, h].sum(0), 0, atol=1e-12)
        live = np.isfinite(LSE[0, h])
        assert np.allclose(dV[0, h].sum(0), dO[0, h][live].sum(0), atol=1e-12)
    cols = np.array([0, 5, 17, 28])
    M = oracle.dense_mask(*v, np.arange(nq))
    _, dkc, dvc = oracle.bwd_rows(Q[0, 1], K[0, 1], V[0, 1], dO[0, 1], M, 0.45, cols=cols)
    assert np.allclose(dkc, dK[0, 1][cols], atol=1e-13) and np.allclose(dvc, dV[0, 1][cols], atol=1e-13)


def test_context_parallel_rows_equal_global_rows():
    """Theorem 1 end to end on tiny sizes: attention of the owned rows with the localised mask
    equals the global-mask attention at those rows."""
    r = rng(8)
    n, d = 48, 4
    L = masks.uniform_cut_lengths(r, n, 5)
    v = masks.document(n, L)
    o, Lc = np.array([8, 32]), np.array([8, 8])
    lv = oracle.localize(*v, o, Lc, n)
    owned = np.concatenate([np.arange(8, 16), np.arange(32, 40)])
    Q, K, V = rand(r, 1, 1, n, d), rand(r, 1, 1, n, d), rand(r, 1, 1, n, d)
    Og, Lg = oracle.attention_fwd(Q, K, V, v, 0.5)
    Ol, Ll = oracle.attention_fwd(Q[:, :, owned], K, V, lv[:4], 0.5)
    assert np.allclose(Ol, Og[:, :, owned], atol=1e-14)
    assert np.array_equal(np.isneginf(Ll), np.isneginf(Lg[:, :, owned]))
