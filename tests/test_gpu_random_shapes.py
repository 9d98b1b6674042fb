"""Seeded random sweep of small problems through flashmask_fwd_ex / flashmask_bwd_ex against the
float64 oracle: random batch and head counts, grouped key/value heads (G = 1..3), any nq, nk in
1..419 (square shapes also draw the structured mask families), both built dtypes.  Each case is
its own test so a failure names its seed.  Bars as elsewhere: O, dQ within 2e-2 (bf16) or 1e-4
(fp32), LSE within 1e-3 with identical -inf rows, and a grouped dK / dV (a sum of G per-head
gradients, formed in float32 and rounded once) within the same bar.  Where an exact bf16
gradient reaches 4 or more, dO is scaled by a power of two first (exact in bf16, so the oracle's
gradients scale by the same factor): values of 8 and more cannot be stored in bf16 within 2e-2.
FM_RANDOM_CASES sets the number of cases (default 24); the first cases of a longer sweep are the
default ones."""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, TOL_LSE, assert_close, dev_i32, f64
from workloads import masks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    import mask_aware_flashattention_amd as m
    m.load_library()
    return m


def draw(case):
    r = np.random.default_rng(np.random.SeedSequence([777, case]))
    dtype = "bf16" if r.random() < 0.8 else "fp32"
    B, Hkv, G = int(r.integers(1, 3)), int(r.integers(1, 3)), int(r.integers(1, 4))
    square = r.random() < 0.6
    nq = int(r.integers(1, 420))
    nk = nq if square else int(r.integers(1, 420))
    kinds = ["random", "none"] + (["causal", "swa", "document", "prefix"] if square else [])
    kind = kinds[int(r.integers(0, len(kinds)))]
    if kind == "random":
        v = masks.random_vectors(r, nk, nq, spread=20)
    elif kind == "none":
        v = masks.no_mask(nk, nq)
    elif kind == "causal":
        v = masks.causal(nk)
    elif kind == "swa":
        v = masks.sliding_window(nk, int(r.integers(1, nk + 1)))
    elif kind == "document":
        v = masks.document(nk, masks.uniform_cut_lengths(r, nk, min(int(r.integers(1, 6)), nk)))
    else:
        v = masks.prefix_lm(nk, int(r.integers(1, nk + 1)))
    return dtype, B, Hkv, G, nq, nk, kind, v


@pytest.mark.parametrize("case", range(int(os.environ.get("FM_RANDOM_CASES", "24"))))
def test_random_shape(fm, case):
    dtype, B, Hkv, G, nq, nk, kind, v = draw(case)
    H = Hkv * G
    d = 128 if dtype == "bf16" else 64
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"random case {case}: {dtype} B={B} H={H} H_kv={Hkv} nq={nq} nk={nk} mask={kind}",
          flush=True)
    g = torch.Generator().manual_seed(case)
    q = torch.randn(B, H, nq, d, generator=g)
    do = torch.randn(B, H, nq, d, generator=g)
    k = torch.randn(B, Hkv, nk, d, generator=g)
    vv = torch.randn(B, Hkv, nk, d, generator=g)
    # keep each dV_j (a sum over up to G*nq/nk rows of dO) where bf16 resolves the bar
    do = do * min(1.0, 2.0 / math.sqrt(max(1.0, G * nq / nk)))
    q, k, vv, do = (x.to(td) for x in (q, k, vv, do))
    scale = 1.0 / math.sqrt(d)
    dvec = [dev_i32(x) for x in v]
    kr, vr = k.repeat_interleave(G, dim=1), vv.repeat_interleave(G, dim=1)
    O, LSE = oracle.attention_fwd(q, kr, vr, v, np.float32(scale))
    dQ, dK, dV = oracle.attention_bwd(q, kr, vr, do, v, np.float32(scale))
    dK = dK.reshape(B, Hkv, G, nk, d).sum(axis=2)
    dV = dV.reshape(B, Hkv, G, nk, d).sum(axis=2)
    if dtype == "bf16":
        # The gradients are linear in dO.  Where one reaches 4 or more (a document's first key
        # collects most of its rows' dO, summed over G heads), dO is scaled by a power of two
        # that brings every gradient below 4, where bf16 storage (spacing 2^-6 .. 2^-5 below 8)
        # resolves the bar; a power of two scales the bf16 dO exactly, so the oracle's
        # gradients scale exactly by the same factor.
        peak = max(np.abs(dQ).max(initial=0.0), np.abs(dK).max(initial=0.0),
                   np.abs(dV).max(initial=0.0))
        if peak >= 4.0:
            c = 2.0 ** -math.ceil(math.log2(peak / 4.0) + 1e-12)
            do = (do.float() * c).to(td)
            dQ, dK, dV = dQ * c, dK * c, dV * c
    qd, kd, vd, dod = (x.cuda() for x in (q, k, vv, do))
    o, lse = fm.fwd_ex(qd, kd, vd, *dvec, scale)
    dq, dk, dvv = fm.bwd_ex(qd, kd, vd, o, dod, lse, *dvec, scale)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    got_lse = f64(lse)
    assert np.array_equal(np.isneginf(got_lse), np.isneginf(LSE)), "LSE: -inf rows differ"
    fin = np.isfinite(LSE)
    if fin.any():
        assert np.abs(got_lse[fin] - LSE[fin]).max() <= TOL_LSE
    for name, got, want in (("O", o, O), ("dQ", dq, dQ), ("dK", dk, dK), ("dV", dvv, dV)):
        assert_close(f"random {dtype} {name}", f64(got), want, tol)
