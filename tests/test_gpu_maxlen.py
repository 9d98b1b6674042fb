"""The longest sequence the tile lists allow: nq = nk = 2^22 - 128 (the forward's 128 x 64 and the
backward's 64 x 128 tile grids then hold just under 2^31 tiles), one head, d = 128, bf16, under a
sliding window of 256 keys.  Rows and key columns near both ends and in the middle are compared
with the oracle on the exact sub-problem (a row only sees the 256 keys before it; a key is only
seen by the 256 rows after it), which also exercises the 32-bit buffer offsets at their largest.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.parity import (TOL, TOL_LSE, assert_close, assert_lse, cols_reference, f64,
                          rows_reference)
from workloads import masks

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

N = (1 << 22) - 128
W = 256


@pytest.fixture(scope="module")
def fm():
    import mask_aware_flashattention_amd as m
    m.load_library()
    return m


def test_max_length_sliding_window(fm):
    vec = masks.sliding_window(N, W)
    gv = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda() for x in vec]
    g = torch.Generator(device="cuda").manual_seed(4194176)
    q, k, v, do = (torch.randn((1, 1, N, 128), generator=g, device="cuda").to(torch.bfloat16)
                   for _ in range(4))
    scale = float(np.float32(1.0 / np.sqrt(128)))
    o, lse = fm.fwd(q, k, v, *gv, scale)
    dq, dk, dv = fm.bwd(q, k, v, o, do, lse, *gv, scale)
    torch.cuda.synchronize()

    def rows_of(t, a, b):
        return f64(t[0, 0, a:b])

    tol = TOL["bf16"]
    for i in (0, 1, W - 1, W, N // 2, N - W, N - 1):
        k0 = max(0, i - W + 1)
        sub = [x[k0:i + 1] for x in vec]
        M = oracle.dense_mask(*sub, [i])
        O, LSE = oracle.fwd_rows(rows_of(q, i, i + 1), rows_of(k, k0, i + 1),
                                 rows_of(v, k0, i + 1), M, scale)
        dQ, _, _ = oracle.bwd_rows(rows_of(q, i, i + 1), rows_of(k, k0, i + 1),
                                   rows_of(v, k0, i + 1), rows_of(do, i, i + 1), M, scale,
                                   cols=np.zeros(0, dtype=np.int64))
        assert np.abs(rows_of(o, i, i + 1) - O).max() <= tol, i
        assert abs(float(lse[0, 0, i]) - LSE[0]) <= TOL_LSE, i
        assert np.abs(rows_of(dq, i, i + 1) - dQ).max() <= tol, i
    for j in (0, 1, N // 2, N - 2, N - 1):
        r0, r1 = j, min(N, j + W)              # rows that see key j
        k0, k1 = max(0, r0 - W + 1), r1        # keys those rows see
        sub = [x[k0:k1] for x in vec]
        M = oracle.dense_mask(*sub, np.arange(r0, r1))
        _, dK, dV = oracle.bwd_rows(rows_of(q, r0, r1), rows_of(k, k0, k1), rows_of(v, k0, k1),
                                    rows_of(do, r0, r1), M, scale, cols=np.array([j - k0]))
        assert np.abs(rows_of(dk, j, j + 1) - dK).max() <= tol, j
        assert np.abs(rows_of(dv, j, j + 1) - dV).max() <= tol, j


@pytest.mark.parametrize("dt,w", [("bf16", 1), ("bf16", 64), ("bf16", 200), ("bf16", 300),
                                  ("fp32", 1), ("fp32", 200)])
def test_long_query_short_walks(fm, dt, w):
    """nq >= 65536 selects the dK/dV kernel's 8-wave shape (128-key column blocks, three tile
    buffers); a sliding window of w keys gives every key block a walk of 2 to 7 query tiles, so
    the start of its pipeline, the three-buffer rotation and both remainders run at that shape.
    nq = nk = 65536 + 77 leaves a ragged last block in both directions.  bf16 runs at d = 128,
    float32 at d = 64."""
    n = 65536 + 77
    d, dtype = (128, torch.bfloat16) if dt == "bf16" else (64, torch.float32)
    vec = masks.sliding_window(n, w)
    gv = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda() for x in vec]
    g = torch.Generator(device="cuda").manual_seed(w)
    q, k, v, do = (torch.randn((1, 1, n, d), generator=g, device="cuda").to(dtype)
                   for _ in range(4))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    print(f"long query, {dt}, window {w}", flush=True)
    o, lse = fm.fwd(q, k, v, *gv, scale)
    dq, dk, dv = fm.bwd(q, k, v, o, do, lse, *gv, scale)
    torch.cuda.synchronize()

    def rows_of(t, a, b):
        return f64(t[0, 0, a:b])

    tol = TOL[dt]
    for i in (0, w, 4097, n // 2 + 3, n - 1):
        k0 = max(0, i - w + 1)
        sub = [x[k0:i + 1] for x in vec]
        M = oracle.dense_mask(*sub, [i])
        dQ, _, _ = oracle.bwd_rows(rows_of(q, i, i + 1), rows_of(k, k0, i + 1),
                                   rows_of(v, k0, i + 1), rows_of(do, i, i + 1), M, scale,
                                   cols=np.zeros(0, dtype=np.int64))
        assert np.abs(rows_of(dq, i, i + 1) - dQ).max() <= tol, i
    for j in (0, 127, 128, 4095, n // 2, n - 78, n - 1):
        r0, r1 = j, min(n, j + w)              # rows that see key j
        k0, k1 = max(0, r0 - w + 1), r1        # keys those rows see
        sub = [x[k0:k1] for x in vec]
        M = oracle.dense_mask(*sub, np.arange(r0, r1))
        _, dK, dV = oracle.bwd_rows(rows_of(q, r0, r1), rows_of(k, k0, k1), rows_of(v, k0, k1),
                                    rows_of(do, r0, r1), M, scale, cols=np.array([j - k0]))
        assert np.abs(rows_of(dk, j, j + 1) - dK).max() <= tol, j
        assert np.abs(rows_of(dv, j, j + 1) - dV).max() <= tol, j


def test_long_query_grouped_heads_with_per_head_masks(fm):
    """The grouped-head (G > 1) instantiation of the dK/dV kernel's 8-wave shape (nq >= 65536,
    three tile buffers), which walks the tile lists of a group's query heads as one sequence and
    points rows past nq at the buffer end: H = 4 query heads over H_kv = 2 key/value heads, one
    mask set per head, and in the first group a head whose every list is empty (every key fully
    masked), so the walk moves from a head with tiles across one without any.  nq = nk =
    65536 + 77 leaves ragged last blocks.  Sampled rows (O, LSE, dQ) per query head and sampled
    key columns (dK, dV summed over the group's heads) against the oracle on exact
    sub-problems; every output against per-head plain calls on the same data."""
    n, d, H, H_kv = 65536 + 77, 128, 4, 2
    G = H // H_kv
    r = np.random.default_rng(np.random.SeedSequence([65613, 4]))
    full = (np.zeros(n, np.int32), np.full(n, n, np.int32), np.zeros(n, np.int32),
            np.zeros(n, np.int32))
    sets = [masks.sliding_window(n, 300), full, masks.sliding_window(n, 2000),
            masks.document(n, masks.uniform_cut_lengths(r, n, 48))]
    vec = [torch.from_numpy(np.ascontiguousarray(np.stack([s_[i] for s_ in sets]))).cuda()
           for i in range(4)]                                          # [H, nk] each
    g = torch.Generator(device="cuda").manual_seed(4242)
    q, do = (torch.randn((1, H, n, d), generator=g, device="cuda").to(torch.bfloat16)
             for _ in range(2))
    k, v = (torch.randn((1, H_kv, n, d), generator=g, device="cuda").to(torch.bfloat16)
            for _ in range(2))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    print("long query, grouped heads H=4 H_kv=2, per-head masks (one head fully masked)",
          flush=True)
    o, lse = fm.fwd_ex(q, k, v, *vec, scale)
    dq, dk, dv = fm.bwd_ex(q, k, v, o, do, lse, *vec, scale)
    torch.cuda.synchronize()
    # per-head plain calls: O, LSE, dQ bit for bit; grouped dK, dV within the bf16 bound of
    # the per-head sums
    dk_sum = torch.zeros(1, H_kv, n, d, device="cuda")
    dv_sum, dk_abs, dv_abs = (torch.zeros_like(dk_sum) for _ in range(3))
    for h in range(H):
        hk = h // G
        sv = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in sets[h]]
        qs, dos = q[:, h:h + 1].contiguous(), do[:, h:h + 1].contiguous()
        ks, vs = k[:, hk:hk + 1].contiguous(), v[:, hk:hk + 1].contiguous()
        o1, lse1 = fm.fwd(qs, ks, vs, *sv, scale)
        dq1, dk1, dv1 = fm.bwd(qs, ks, vs, o1, dos, lse1, *sv, scale)
        torch.cuda.synchronize()
        assert torch.equal(o[:, h:h + 1], o1) and torch.equal(lse[:, h:h + 1], lse1), h
        assert torch.equal(dq[:, h:h + 1], dq1), h
        dk_sum[:, hk] += dk1[:, 0].float()
        dv_sum[:, hk] += dv1[:, 0].float()
        dk_abs[:, hk] += dk1[:, 0].float().abs()
        dv_abs[:, hk] += dv1[:, 0].float().abs()
    assert not dq[:, 1].any() and bool(torch.isneginf(lse[:, 1]).all())
    for got, ref, absum in ((dk, dk_sum, dk_abs), (dv, dv_sum, dv_abs)):
        err = (got.float() - ref).abs()
        assert bool((err <= 2.0 ** -8 * (absum + ref.abs()) * 1.01 + 1e-5).all())
    # the oracle on exact sub-problems
    tol = TOL["bf16"]
    q64 = [f64(q[0, h]) for h in range(H)]
    do64 = [f64(do[0, h]) for h in range(H)]
    k64 = [f64(k[0, hk]) for hk in range(H_kv)]
    v64 = [f64(v[0, hk]) for hk in range(H_kv)]
    rows = np.array([0, 1, 299, 300, 4097, n // 2 + 3, n - 78, n - 1])
    for h in range(H):
        hk = h // G
        O, LSE, dQ = rows_reference(q64[h], k64[hk], v64[hk], do64[h], sets[h], rows, rows,
                                    scale)
        assert_close(f"O h={h}", f64(o[0, h, rows]), O, tol)
        assert_lse(f64(lse[0, h, rows]), LSE)
        assert_close(f"dQ h={h}", f64(dq[0, h, rows]), dQ, tol)
    cols = np.array([0, 127, 128, 4095, n // 2, n - 78, n - 1])
    for hk in range(H_kv):
        dK = np.zeros((len(cols), d))
        dV = np.zeros((len(cols), d))
        for h in range(hk * G, (hk + 1) * G):
            a, b = cols_reference(q64[h], k64[hk], v64[hk], do64[h], sets[h], cols,
                                  np.arange(n), scale)
            dK += a
            dV += b
        assert_close(f"dK group {hk}", f64(dk[0, hk, cols]), dK, tol)
        assert_close(f"dV group {hk}", f64(dv[0, hk, cols]), dV, tol)
