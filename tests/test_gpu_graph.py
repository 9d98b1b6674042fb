"""The forward and backward calls inside a captured HIP graph (torch.cuda.graph): each call only
launches kernels on the caller's stream (no allocation when the workspaces and outputs are
given, no memset, no host synchronisation), so one capture of fwd + bwd (and of the
no-allocation forward) replays to results bit-identical to eager calls on the same inputs:
replayed several times with eager work and synchronisations in between, and again after new
values (inputs and mask vectors) are copied into the captured buffers.  The kernels use no
atomics, so equal inputs give equal bits."""

import numpy as np
import pytest
import torch

from tests.parity import dev_i32
from workloads import masks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    import mask_aware_flashattention_amd as m
    m.load_library()
    return m


def _vectors(seed, n, docs):
    r = np.random.default_rng(np.random.SeedSequence([3, seed]))
    return [dev_i32(x) for x in masks.document(n, masks.uniform_cut_lengths(r, n, docs))]


def _eager(fm, q, k, v, do, vec, scale):
    o, lse = fm.fwd(q, k, v, *vec, scale)
    dq, dk, dv = fm.bwd(q, k, v, o, do, lse, *vec, scale)
    o_na = torch.empty_like(q)
    lse_na = torch.empty_like(lse)
    fm.fwd_noalloc(q, k, v, *vec, scale, out=o_na, lse=lse_na)
    return [o, lse, dq, dk, dv, o_na, lse_na]


def test_graph_replays_match_eager(fm):
    B, H, n, d = 1, 2, 1000, 128
    scale = float(np.float32(1.0 / np.sqrt(d)))
    g = torch.Generator(device="cuda").manual_seed(11)
    q, k, v, do = (torch.randn((B, H, n, d), generator=g, device="cuda").to(torch.bfloat16)
                   for _ in range(4))
    vec = _vectors(0, n, 5)
    shape_args = (q, k, v)
    from mask_aware_flashattention_amd import _lib
    shp = _lib.FmShape(B, H, n, n, d, _lib.FM_BF16)
    ws_f = torch.empty(fm.fwd_workspace_bytes(shp), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(fm.bwd_workspace_bytes(shp), dtype=torch.uint8, device="cuda")
    o, dq, dk, dv, o_na = (torch.empty_like(q) for _ in range(5))
    lse, lse_na = (torch.empty((B, H, n), dtype=torch.float32, device="cuda") for _ in range(2))
    outs = [o, lse, dq, dk, dv, o_na, lse_na]

    def step():
        fm.fwd(*shape_args, *vec, scale, out=o, lse=lse, workspace=ws_f)
        fm.bwd(*shape_args, o, do, lse, *vec, scale, workspace=ws_b, grads=(dq, dk, dv))
        fm.fwd_noalloc(*shape_args, *vec, scale, out=o_na, lse=lse_na)

    # warm-up on a side stream (also sets up the no-allocation array), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    def check(tag):
        want = _eager(fm, q, k, v, do, vec, scale)
        torch.cuda.synchronize()
        for name, got, ref in zip(["O", "LSE", "dQ", "dK", "dV", "O noalloc", "LSE noalloc"],
                                  outs, want):
            assert torch.equal(got, ref), f"{tag}: {name} differs from the eager call"

    print("graph capture: replays against eager calls", flush=True)
    for rep in range(3):
        for t in outs:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        check(f"replay {rep}")
        # eager work of the program's own between replays
        x = torch.randn(512, 512, device="cuda")
        (x @ x).sum().item()

    # new values in the captured buffers: inputs and the mask vectors
    for t in (q, k, v, do):
        t.copy_(torch.randn(t.shape, generator=g, device="cuda").to(t.dtype))
    for dst, src in zip(vec, _vectors(1, n, 9)):
        dst.copy_(src)
    graph.replay()
    torch.cuda.synchronize()
    check("replay with new inputs and mask")
