"""GPU parity of the interface variants (flashmask_fwd_ex / flashmask_bwd_ex): strided tensors,
grouped key/value heads and per-batch / per-head mask vectors.

* A variant only changes which memory a (batch, head) reads, so its outputs must equal, bit for
  bit, the plain calls on the same per-(batch, head) data: strided views against contiguous
  copies; grouped heads against K/V repeated for every query head (O, LSE, dQ); per-head and
  per-batch vectors against one plain call per (batch, head).
* dK and dV of a grouped key/value head are the sum of its G query heads' gradients, formed in
  float32 and rounded to bf16 once; against the bf16 per-head results of the repeated run the
  difference is at most 2^-8 (sum of |parts| + |result|) plus float32 reordering.
* Against the float64 oracle, applied per (batch, head) with that head's key/value head and mask
  set: O, dQ within 2e-2, LSE within 1e-3; a grouped dK / dV against the sum of its G heads'
  oracle gradients within the same 2e-2 (the kernel sums the G heads in float32 and rounds
  once).  dO is scaled by 1 / sqrt(G) so that the grouped sums (about sqrt(G) times one head's
  gradient) stay below 8, where bf16 storage resolves 2e-2.
"""

import math

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


def rng(*k):
    return np.random.default_rng(np.random.SeedSequence([91, *k]))


def randn(g, *shape):
    return torch.randn(*shape, generator=g).to(torch.bfloat16).cuda()


def stack_sets(sets):
    """[sets...] of 4-vector tuples -> four int32 device tensors shaped like the set grid."""
    arr = np.asarray(sets, dtype=np.int32)          # [..., 4, nk]
    return [dev_i32(np.ascontiguousarray(arr[..., i, :])) for i in range(4)]


def mask_for(r, kind, n):
    if kind == "document":
        return masks.document(n, masks.uniform_cut_lengths(r, n, int(r.integers(2, 6))))
    if kind == "swa":
        return masks.sliding_window(n, int(r.integers(16, n)))
    if kind == "causal":
        return masks.causal(n)
    if kind == "random":
        return masks.random_vectors(r, n, n, spread=20)
    if kind == "all":
        return (np.zeros(n, np.int32), np.full(n, n, np.int32), np.zeros(n, np.int32),
                np.zeros(n, np.int32))
    raise ValueError(kind)


def bf16_sum_bound(parts_abs, ref):
    return 2.0 ** -8 * (parts_abs + ref.abs()) * 1.01 + 1e-5


def test_strided_views_equal_contiguous_calls(fm):
    B, H, n, d = 2, 4, 523, 128
    r = rng(1)
    vec = [dev_i32(x) for x in mask_for(r, "document", n)]
    g = torch.Generator().manual_seed(11)
    # packed [B, n, 3, H, d] (one projection output): q, k, v are strided views of it
    qkv = randn(g, B, n, 3, H, d)
    q, k, v = (qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    do_full = randn(g, B, n, 3, H, d)
    do = do_full[:, :, 0].permute(0, 2, 1, 3)
    assert not q.is_contiguous() and do.stride() == q.stride()
    print("strided views: B=2 H=4 n=523 rows of 3*H*d", flush=True)
    o_x, lse_x = fm.fwd_ex(q, k, v, *vec)
    dq_x, dk_x, dv_x = fm.bwd_ex(q, k, v, o_x, do, lse_x, *vec)
    qc, kc, vc, doc = (t.contiguous() for t in (q, k, v, do))
    o, lse = fm.fwd(qc, kc, vc, *vec)
    dq, dk, dv = fm.bwd(qc, kc, vc, o, doc, lse, *vec)
    torch.cuda.synchronize()
    assert o_x.stride() == q.stride() and dq_x.stride() == q.stride() and dk_x.stride() == k.stride()
    for name, a, b in (("O", o_x, o), ("LSE", lse_x, lse), ("dQ", dq_x, dq), ("dK", dk_x, dk),
                       ("dV", dv_x, dv)):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("H,H_kv,kind", [(4, 2, "causal"), (4, 1, "random"), (6, 3, "swa"),
                                         (8, 1, "document")])
def test_grouped_heads(fm, H, H_kv, kind):
    B, n, d = 1, 389, 128
    G = H // H_kv
    r = rng(2, H, H_kv)
    vec_np = mask_for(r, kind, n)
    vec = [dev_i32(x) for x in vec_np]
    g = torch.Generator().manual_seed(12 + H)
    q, do = randn(g, B, H, n, d), randn(g, B, H, n, d)
    k, v = randn(g, B, H_kv, n, d), randn(g, B, H_kv, n, d)
    do = (do.float() / math.sqrt(G)).to(torch.bfloat16)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    print(f"grouped heads H={H} H_kv={H_kv} mask={kind}", flush=True)
    o_x, lse_x = fm.fwd_ex(q, k, v, *vec, scale)
    dq_x, dk_x, dv_x = fm.bwd_ex(q, k, v, o_x, do, lse_x, *vec, scale)
    kr, vr = k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1)
    o, lse = fm.fwd(q, kr, vr, *vec, scale)
    dq, dk, dv = fm.bwd(q, kr, vr, o, do, lse, *vec, scale)
    torch.cuda.synchronize()
    assert torch.equal(o_x, o) and torch.equal(lse_x, lse) and torch.equal(dq_x, dq)
    for got, per_head in ((dk_x, dk), (dv_x, dv)):
        parts = per_head.float().view(B, H_kv, G, n, d)
        ref = parts.sum(dim=2)
        err = (got.float() - ref).abs()
        assert bool((err <= bf16_sum_bound(parts.abs().sum(dim=2), ref)).all())
    # oracle, per query head against its key/value head
    qn, kn, vn, don = (f64(t) for t in (q, k, v, do))
    dK = np.zeros((B, H_kv, n, d))
    dV = np.zeros((B, H_kv, n, d))
    for h in range(H):
        hk = h // G
        O, LSE = oracle.attention_fwd(qn[:, h:h + 1], kn[:, hk:hk + 1], vn[:, hk:hk + 1], vec_np, np.float32(scale))
        dQ, dKh, dVh = oracle.attention_bwd(qn[:, h:h + 1], kn[:, hk:hk + 1], vn[:, hk:hk + 1],
                                            don[:, h:h + 1], vec_np, np.float32(scale))
        assert np.abs(f64(o_x[:, h:h + 1]) - O).max() <= TOL["bf16"], h
        live = ~np.isneginf(LSE)
        assert np.abs(f64(lse_x[:, h:h + 1])[live] - LSE[live]).max() <= TOL_LSE, h
        assert np.abs(f64(dq_x[:, h:h + 1]) - dQ).max() <= TOL["bf16"], h
        dK[:, hk:hk + 1] += dKh
        dV[:, hk:hk + 1] += dVh
    assert_close(f"grouped dK G={G}", f64(dk_x), dK, TOL["bf16"])
    assert_close(f"grouped dV G={G}", f64(dv_x), dV, TOL["bf16"])


@pytest.mark.parametrize("mask_b,mask_h,H_kv", [(1, 4, 4), (2, 1, 4), (2, 4, 4), (2, 4, 2)])
def test_mask_sets(fm, mask_b, mask_h, H_kv):
    """Per-batch and per-head vectors (one set fully masked), with and without grouped heads."""
    B, H, n, d = 2, 4, 457, 128
    G = H // H_kv
    r = rng(3, mask_b, mask_h, H_kv)
    kinds = ["document", "all", "causal", "swa", "random", "document", "causal", "swa"]
    sets = [[mask_for(r, kinds[(b * mask_h + h) % len(kinds)], n) for h in range(mask_h)]
            for b in range(mask_b)]
    vec = stack_sets(sets)                       # each [mask_b, mask_h, nk]
    g = torch.Generator().manual_seed(13 + mask_b * 7 + mask_h + H_kv)
    q, do = randn(g, B, H, n, d), randn(g, B, H, n, d)
    k, v = randn(g, B, H_kv, n, d), randn(g, B, H_kv, n, d)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    print(f"mask sets mask_b={mask_b} mask_h={mask_h} H_kv={H_kv}", flush=True)
    o_x, lse_x = fm.fwd_ex(q, k, v, *vec, scale)
    dq_x, dk_x, dv_x = fm.bwd_ex(q, k, v, o_x, do, lse_x, *vec, scale)
    torch.cuda.synchronize()
    dk_sum = torch.zeros(B, H_kv, n, d, device="cuda")
    dv_sum = torch.zeros_like(dk_sum)
    dk_abs, dv_abs = torch.zeros_like(dk_sum), torch.zeros_like(dk_sum)
    for b in range(B):
        for h in range(H):
            hk = h // G
            s = sets[b if mask_b > 1 else 0][h if mask_h > 1 else 0]
            sv = [dev_i32(x) for x in s]
            qs, dos = q[b:b + 1, h:h + 1].contiguous(), do[b:b + 1, h:h + 1].contiguous()
            ks, vs = k[b:b + 1, hk:hk + 1].contiguous(), v[b:b + 1, hk:hk + 1].contiguous()
            o, lse = fm.fwd(qs, ks, vs, *sv, scale)
            dq, dk, dv = fm.bwd(qs, ks, vs, o, dos, lse, *sv, scale)
            torch.cuda.synchronize()
            assert torch.equal(o_x[b:b + 1, h:h + 1], o), (b, h)
            assert torch.equal(lse_x[b:b + 1, h:h + 1], lse), (b, h)
            assert torch.equal(dq_x[b:b + 1, h:h + 1], dq), (b, h)
            if G == 1:
                assert torch.equal(dk_x[b:b + 1, hk:hk + 1], dk), (b, h)
                assert torch.equal(dv_x[b:b + 1, hk:hk + 1], dv), (b, h)
            dk_sum[b, hk] += dk[0, 0].float()
            dv_sum[b, hk] += dv[0, 0].float()
            dk_abs[b, hk] += dk[0, 0].float().abs()
            dv_abs[b, hk] += dv[0, 0].float().abs()
            # oracle on this (batch, head)
            O, LSE = oracle.attention_fwd(f64(qs), f64(ks), f64(vs), s, np.float32(scale))
            assert np.abs(f64(o) - O).max() <= TOL["bf16"], (b, h)
            live = ~np.isneginf(LSE)
            assert np.array_equal(np.isneginf(f64(lse)), ~live), (b, h)
            if live.any():
                assert np.abs(f64(lse)[live] - LSE[live]).max() <= TOL_LSE, (b, h)
    for got, ref, absum in ((dk_x, dk_sum, dk_abs), (dv_x, dv_sum, dv_abs)):
        err = (got.float() - ref).abs()
        assert bool((err <= bf16_sum_bound(absum, ref)).all())


def test_everything_at_once(fm):
    """Strided packed Q/K/V, grouped heads and per-head masks together, against per-head plain
    calls on contiguous copies."""
    B, H, H_kv, n, d = 2, 4, 2, 301, 128
    G = H // H_kv
    r = rng(4)
    sets = [[mask_for(r, k, n) for k in ("document", "swa", "all", "random")]]
    vec = stack_sets(sets)                       # [1, H, nk]
    g = torch.Generator().manual_seed(14)
    packed = randn(g, B, n, H + 2 * H_kv, d)     # [B, n, heads of q | k | v, d]
    q = packed[:, :, :H].permute(0, 2, 1, 3)
    k = packed[:, :, H:H + H_kv].permute(0, 2, 1, 3)
    v = packed[:, :, H + H_kv:].permute(0, 2, 1, 3)
    do = randn(g, B, n, H + 2 * H_kv, d)[:, :, :H].permute(0, 2, 1, 3)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    print("strided + grouped + per-head masks", flush=True)
    o_x, lse_x = fm.fwd_ex(q, k, v, *vec, scale)
    dq_x, dk_x, dv_x = fm.bwd_ex(q, k, v, o_x, do, lse_x, *vec, scale)
    dk_sum = torch.zeros(B, H_kv, n, d, device="cuda")
    dv_sum, dk_abs, dv_abs = (torch.zeros_like(dk_sum) for _ in range(3))
    for b in range(B):
        for h in range(H):
            hk = h // G
            sv = [dev_i32(x) for x in sets[0][h]]
            qs, dos = q[b:b + 1, h:h + 1].contiguous(), do[b:b + 1, h:h + 1].contiguous()
            ks, vs = k[b:b + 1, hk:hk + 1].contiguous(), v[b:b + 1, hk:hk + 1].contiguous()
            o, lse = fm.fwd(qs, ks, vs, *sv, scale)
            dq, dk, dv = fm.bwd(qs, ks, vs, o, dos, lse, *sv, scale)
            torch.cuda.synchronize()
            assert torch.equal(o_x[b:b + 1, h:h + 1], o), (b, h)
            assert torch.equal(lse_x[b:b + 1, h:h + 1], lse), (b, h)
            assert torch.equal(dq_x[b:b + 1, h:h + 1], dq), (b, h)
            dk_sum[b, hk] += dk[0, 0].float()
            dv_sum[b, hk] += dv[0, 0].float()
            dk_abs[b, hk] += dk[0, 0].float().abs()
            dv_abs[b, hk] += dv[0, 0].float().abs()
    for got, ref, absum in ((dk_x, dk_sum, dk_abs), (dv_x, dv_sum, dv_abs)):
        err = (got.float() - ref).abs()
        assert bool((err <= bf16_sum_bound(absum, ref)).all())
