"""GPU parity of the integer kernels (bit-exact against the oracle): clip-shift-max
localisation and tile classification with list compaction."""

import numpy as np
import pytest
import torch

import oracle
from tests.parity import dev_i32
from workloads import configs, masks

pytestmark = pytest.mark.gpu

I32_MIN, I32_MAX = np.iinfo(np.int32).min, np.iinfo(np.int32).max


@pytest.fixture(scope="module")
def fm():
    import mask_aware_flashattention_amd as m
    m.load_library()
    return m


def rng(*k):
    return np.random.default_rng(np.random.SeedSequence([11, *k]))


def run_localize(fm, vecs, starts, lens, nq_global, offset=0):
    # offset > 0 views the vectors at a 4-byte (not 16-byte) aligned address
    dev = [torch.zeros(len(v) + offset, dtype=torch.int32, device="cuda") for v in vecs]
    for d, v in zip(dev, vecs):
        d[offset:] = dev_i32(v)
    views = [d[offset:] for d in dev]
    out = fm.localize(*views, starts, lens, nq_global)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out[:4]], out[4]


def test_localize_cp_share(fm):
    w = configs.WORKLOADS["c5"]
    v = configs.global_mask(w)
    got, n_local = run_localize(fm, v, configs.C5_CHUNK_START, configs.C5_CHUNK_LEN, 131072)
    want = oracle.localize(*v, configs.C5_CHUNK_START, configs.C5_CHUNK_LEN, 131072)
    assert n_local == want[4] == 8192
    for a, b in zip(got, want[:4]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("seed", range(12))
def test_localize_random(fm, seed):
    r = rng(1, seed)
    n = int(r.choice([1, 3, 4, 5, 64, 1000, 4097, 65536 + 3]))
    nq_global = int(r.integers(1, 1 << 20))
    k = int(r.integers(1, min(64, (nq_global + 1) // 2) + 1))
    pts = np.sort(r.choice(nq_global + 1, size=2 * k, replace=False))
    starts, lens = pts[0::2], pts[1::2] - pts[0::2]
    vecs = [r.integers(-nq_global // 4, nq_global + nq_global // 4, size=n, dtype=np.int64)
            .astype(np.int32) for _ in range(4)]
    vecs[0][: min(n, 2)] = [I32_MIN, I32_MAX][: min(n, 2)]
    offset = int(seed % 2)
    print(f"localize seed={seed} n={n} chunks={k} offset={offset}", flush=True)
    got, n_local = run_localize(fm, vecs, starts, lens, nq_global, offset)
    want = oracle.localize(*vecs, starts, lens, nq_global)
    assert n_local == want[4]
    for a, b in zip(got, want[:4]):
        assert np.array_equal(a, b)


def compare_classify(got, want, BM, BN):
    cls = got["cls"].cpu().numpy()
    assert np.array_equal(cls, want["cls"])
    qcnt, qlist = got["qcnt"].cpu().numpy(), got["qlist"].cpu().numpy()
    kcnt, klist = got["kcnt"].cpu().numpy(), got["klist"].cpu().numpy()
    assert np.array_equal(qcnt, want["qcnt"])
    assert np.array_equal(kcnt, want["kcnt"])
    for qb, lst in enumerate(want["qlist"]):
        assert np.array_equal(qlist[qb, :len(lst)], lst), qb
    for kb, lst in enumerate(want["klist"]):
        assert np.array_equal(klist[kb, :len(lst)], lst), kb


@pytest.mark.parametrize("key", ["c1", "c2a", "c2b", "c2c", "c2d", "c2e", "c2f", "c3", "c3m", "c5"])
def test_classify_workloads_at_kernel_tiles(fm, key):
    w = configs.WORKLOADS[key]
    v = configs.global_mask(w)
    if key == "c5":
        v = oracle.localize(*v, configs.C5_CHUNK_START, configs.C5_CHUNK_LEN, 131072)[:4]
    dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    bm_f, bn_f, bm_b, bn_b = fm.tile_sizes(dtype, w.d)
    dv = [dev_i32(x) for x in v]
    for BM, BN in ((bm_f, bn_f), (bm_b, bn_b)):
        print(f"classify {key} BM={BM} BN={BN}", flush=True)
        got = fm.classify(*dv, w.nq, BM, BN)
        torch.cuda.synchronize()
        compare_classify(got, oracle.classify(*v, w.nq, BM, BN), BM, BN)


@pytest.mark.parametrize("key", ["c4swa", "c4doc"])
def test_classify_128k_at_both_kernel_grids(fm, key):
    """The 128K masks at the tile grids the attention calls really walk there: the forward and
    dQ kernels' row lists at BM_fwd x BN_fwd, and the dK/dV kernel's column lists at BM_bwd x
    2*BN_bwd (for nq >= 65536 its key blocks are twice as wide)."""
    w = configs.WORKLOADS[key]
    v = configs.global_mask(w)
    bm_f, bn_f, bm_b, bn_b = fm.tile_sizes(torch.bfloat16, w.d)
    assert w.nq >= 65536
    dv = [dev_i32(x) for x in v]
    for BM, BN in ((bm_f, bn_f), (bm_b, 2 * bn_b)):
        print(f"classify {key} BM={BM} BN={BN}", flush=True)
        got = fm.classify(*dv, w.nq, BM, BN, qlists=True, klists=True)
        torch.cuda.synchronize()
        compare_classify(got, oracle.classify(*v, w.nq, BM, BN), BM, BN)


@pytest.mark.parametrize("seed", range(16))
def test_classify_random_vectors_and_tiles(fm, seed):
    r = rng(2, seed)
    nq, nk = int(r.integers(1, 3000)), int(r.integers(1, 3000))
    BM, BN = int(r.integers(1, 300)), int(r.integers(1, 300))
    v = list(masks.random_vectors(r, nk, nq, spread=int(r.integers(0, 50))))
    if seed % 4 == 0:
        v[1] = np.full(nk, I32_MAX, np.int32)
        v[2] = np.full(nk, I32_MIN, np.int32)
    print(f"classify random seed={seed} nq={nq} nk={nk} BM={BM} BN={BN}", flush=True)
    got = fm.classify(*[dev_i32(x) for x in v], nq, BM, BN)
    torch.cuda.synchronize()
    compare_classify(got, oracle.classify(*v, nq, BM, BN), BM, BN)


@pytest.mark.parametrize("n,top", [(1, 1), (300, 100), (5000, 5000), (65536, 1 << 16), (77, 0)])
def test_block_order_matches_its_definition(fm, n, top):
    # a scheduling aid, not part of the method: compared with its definition in the header
    r = rng(5, n)
    cnt = r.integers(0, top + 1, size=n).astype(np.int32)
    cnt[r.integers(0, n, size=min(n, 7))] = top  # ties at the maximum
    order = fm.api.block_order(dev_i32(cnt)).cpu().numpy()
    bucket = (np.maximum(cnt, 0).astype(np.int64) * 4) // (int(cnt.max()) + 1)
    want = [i for b in (3, 2, 1, 0) for i in range(n - 1, -1, -1) if bucket[i] == b]
    assert np.array_equal(order, np.asarray(want))
