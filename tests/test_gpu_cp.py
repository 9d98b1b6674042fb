"""Context parallelism on one GPU: the key/value chunk prune list, and every rank of a 16-way
share run one after another and put back together.

* Prune list (flashmask_prune_chunks): bit-exact against the oracle on the localised vectors of
  every rank of the 128K context-parallel workload, and on arbitrary vectors and shapes.
* All-ranks emulation: for each of the 16 ranks (row chunks r and 31 - r of 32 chunks of 4096
  rows of the 128K document mask), localise the global vectors, run the forward and the backward
  on the rank's rows against all keys, and reassemble.  By Theorem 1 (FlashMask-3 explainer,
  clip-shift-max paragraph) every local tile has the class of the matching global tile, so the
  local calls walk the same tiles as one global call: O, LSE and dQ must equal the global call's
  bit for bit.  dK and dV are sums of the ranks' bf16 partials; each partial and the global
  result are round-to-nearest bf16 of float32 sums, so the reassembled sum may differ from the
  global dK by at most 2^-8 (sum of |partials| + |global|) plus float32 reordering (bound used
  below).  Chunks that the prune list drops contribute nothing to a rank.
  The reassembled result of head 0 (O, LSE, dQ put back at the ranks' rows; dK and dV summed
  over the ranks) is also compared element by element with the float64 oracle of the global
  problem, every row and every key column.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, assert_close, assert_lse, dev_i32, f64, whole_head_reference
from workloads import configs, masks

pytestmark = pytest.mark.gpu

R, CHUNK = configs.C5_DEGREE, configs.C5_CHUNK   # 16 ranks, 2 x 4096 rows each
N = 2 * R * CHUNK                                   # 131072


@pytest.fixture(scope="module")
def fm():
    import mask_aware_flashattention_amd as m
    m.load_library()
    return m


def rank_chunks(r):
    starts = [r * CHUNK, (2 * R - 1 - r) * CHUNK]
    return starts, [CHUNK, CHUNK]


def rank_rows(r):
    s, L = rank_chunks(r)
    return torch.cat([torch.arange(a, a + b) for a, b in zip(s, L)]).cuda()


@pytest.fixture(scope="module")
def global_vectors():
    w = configs.WORKLOADS["c5"]
    return configs.global_mask(w)


def test_prune_list_every_rank_matches_oracle(fm, global_vectors):
    gv = [dev_i32(x) for x in global_vectors]
    for r in range(R):
        s, L = rank_chunks(r)
        lv = fm.localize(*gv, s, L, N)
        live = fm.prune_chunks(*lv[:4], lv[4], CHUNK, CHUNK).cpu().numpy()
        want_v = oracle.localize(*global_vectors, s, L, N)
        want = oracle.prune_chunks(*want_v[:4], want_v[4], CHUNK, CHUNK)
        assert np.array_equal(live, want), r


@pytest.mark.parametrize("seed", range(8))
def test_prune_list_random(fm, seed):
    r = np.random.default_rng(np.random.SeedSequence([72, seed]))
    n_local = int(r.integers(1, 3000))
    nk = int(r.integers(1, 5000))
    BM = int(r.integers(1, 700))
    chunk = int(r.integers(1, 900))
    v = masks.random_vectors(r, nk, n_local, spread=int(r.integers(0, 40)))
    live = fm.prune_chunks(*[dev_i32(x) for x in v], n_local, BM, chunk).cpu().numpy()
    assert np.array_equal(live, oracle.prune_chunks(*v, n_local, BM, chunk))


def test_all_ranks_reassemble_to_the_global_call(fm, global_vectors):
    B, H, d = 1, 16, 128
    g = torch.Generator(device="cuda").manual_seed(20261203)
    q, k, v, do = (torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
                   for _ in range(4))
    gv = [dev_i32(x) for x in global_vectors]
    o, lse = fm.fwd(q, k, v, *gv)
    dq, dk, dv = fm.bwd(q, k, v, o, do, lse, *gv)

    o_re = torch.zeros_like(o[0, 0])     # head 0 put back together from the ranks
    lse_re = torch.full_like(lse[0, 0], float("nan"))
    dq_re = torch.zeros_like(dq[0, 0])
    dk_sum = torch.zeros_like(dk, dtype=torch.float32)
    dv_sum = torch.zeros_like(dv, dtype=torch.float32)
    dk_abs = torch.zeros_like(dk_sum)
    dv_abs = torch.zeros_like(dv_sum)
    skipped = 0
    for r in range(R):
        s, L = rank_chunks(r)
        rows = rank_rows(r)
        lv = fm.localize(*gv, s, L, N)
        assert lv[4] == 2 * CHUNK
        q_l = q.index_select(2, rows).contiguous()
        do_l = do.index_select(2, rows).contiguous()
        o_l, lse_l = fm.fwd(q_l, k, v, *lv[:4])
        dq_l, dk_r, dv_r = fm.bwd(q_l, k, v, o_l, do_l, lse_l, *lv[:4])
        torch.cuda.synchronize()
        assert torch.equal(o_l, o.index_select(2, rows)), r
        assert torch.equal(lse_l, lse.index_select(2, rows)), r
        assert torch.equal(dq_l, dq.index_select(2, rows)), r
        o_re[rows] = o_l[0, 0]
        lse_re[rows] = lse_l[0, 0]
        dq_re[rows] = dq_l[0, 0]
        # keys of chunks the rank prunes get exactly zero gradient from it
        live = fm.prune_chunks(*lv[:4], lv[4], CHUNK, CHUNK)
        dead = torch.nonzero(live == 0).flatten()
        skipped += int(dead.numel())
        for c in dead.tolist():
            assert not dk_r[:, :, c * CHUNK:(c + 1) * CHUNK].any(), (r, c)
            assert not dv_r[:, :, c * CHUNK:(c + 1) * CHUNK].any(), (r, c)
        dk_sum += dk_r.float()
        dv_sum += dv_r.float()
        dk_abs += dk_r.float().abs()
        dv_abs += dv_r.float().abs()
    assert skipped > 0  # the document mask lets ranks skip chunks
    for got, ref, absum in ((dk_sum, dk.float(), dk_abs), (dv_sum, dv.float(), dv_abs)):
        bound = 2.0 ** -8 * (absum + ref.abs()) * 1.01 + 1e-5
        err = (got - ref).abs()
        assert bool((err <= bound).all()), float((err - bound).max())
    # head 0 of the reassembled result against the oracle of the global problem
    scale = np.float32(1.0 / np.sqrt(d))
    q64, k64, v64, do64 = (f64(x[0, 0]) for x in (q, k, v, do))
    O, LSE, dQ, dK, dV = whole_head_reference(q64, k64, v64, do64, global_vectors, np.arange(N),
                                              scale)
    tol = TOL["bf16"]
    assert_close("cp16 O", f64(o_re), O, tol)
    assert_lse(f64(lse_re), LSE)
    assert_close("cp16 dQ", f64(dq_re), dQ, tol)
    assert_close("cp16 dK (sum over ranks)", f64(dk_sum[0, 0]), dK, tol)
    assert_close("cp16 dV (sum over ranks)", f64(dv_sum[0, 0]), dV, tol)
