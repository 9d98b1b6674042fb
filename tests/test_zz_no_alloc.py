"""The forward entry point that allocates nothing (flashmask_fwd_noalloc), called through the C
ABI: its workspace is the library's fixed device array, so its outputs must equal flashmask_fwd's
(same kernels, caller-supplied workspace) bit for bit.  Two calls in a row, the second on a
smaller problem, check that what the first call left in the shared array does not leak into the
second.  A problem whose workspace exceeds the array is refused before any device work."""

import ctypes
import math

import numpy as np
import pytest
import torch

from mask_aware_flashattention_amd import _lib
from tests.parity import dev_i32
from workloads import masks

pytestmark = pytest.mark.gpu

FM_ERR_SCRATCH = 10


@pytest.fixture(scope="module")
def lib():
    import mask_aware_flashattention_amd as m
    return m.load_library()


def P(t):
    return ctypes.c_void_p(t.data_ptr())


def problem(seed, B, H, n, d=128):
    r = np.random.default_rng(np.random.SeedSequence([2024, seed]))
    vec = [dev_i32(x) for x in masks.document(n, masks.uniform_cut_lengths(r, n, 5))]
    g = torch.Generator(device="cuda").manual_seed(seed)
    q, k, v = (torch.randn((B, H, n, d), generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    return q, k, v, vec


def run_noalloc(lib, q, k, v, vec, scale):
    B, H, n, d = q.shape
    shape = _lib.FmShape(B, H, n, n, d, _lib.FM_BF16)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, n), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.flashmask_fwd_noalloc(ctypes.byref(shape), P(q), P(k), P(v), *[P(x) for x in vec],
                                   ctypes.c_float(scale), P(o), P(lse),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, _lib.strerror(st)
    return o, lse


def run_plain(lib, q, k, v, vec, scale):
    B, H, n, d = q.shape
    shape = _lib.FmShape(B, H, n, n, d, _lib.FM_BF16)
    ws = torch.empty(lib.flashmask_fwd_workspace_bytes(ctypes.byref(shape)), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, n), dtype=torch.float32, device="cuda")
    st = lib.flashmask_fwd(ctypes.byref(shape), P(q), P(k), P(v), *[P(x) for x in vec],
                           ctypes.c_float(scale), P(o), P(lse), P(ws), ws.numel(),
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, _lib.strerror(st)
    return o, lse


def test_noalloc_equals_plain_forward_twice_in_a_row(lib):
    scale = 1.0 / math.sqrt(128)
    # first a larger problem (its lists fill more of the array), then a smaller one
    for seed, (B, H, n) in ((1, (2, 4, 5000)), (2, (1, 2, 777))):
        print(f"no-alloc forward B={B} H={H} n={n}", flush=True)
        q, k, v, vec = problem(seed, B, H, n)
        o_n, lse_n = run_noalloc(lib, q, k, v, vec, scale)
        o_p, lse_p = run_plain(lib, q, k, v, vec, scale)
        torch.cuda.synchronize()
        assert torch.equal(o_n, o_p)
        assert torch.equal(lse_n, lse_p)


def test_noalloc_refuses_problems_beyond_its_array(lib):
    cap = lib.flashmask_fwd_noalloc_max_workspace_bytes()
    assert cap == 16 << 20
    n = 1 << 18  # 2048 x 4096 list entries at 128 x 64 tiles: 32 MiB of lists
    shape = _lib.FmShape(1, 1, n, n, 128, _lib.FM_BF16)
    assert lib.flashmask_fwd_workspace_bytes(ctypes.byref(shape)) > cap
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: the size check comes first
    st = lib.flashmask_fwd_noalloc(ctypes.byref(shape), fake, fake, fake, fake, fake, fake, fake,
                                   ctypes.c_float(0.1), fake, fake, ctypes.c_void_p(0))
    assert st == FM_ERR_SCRATCH
