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
from tests.parity import TOL, TOL_LSE, f64
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
