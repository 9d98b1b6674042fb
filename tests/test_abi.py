"""Host-side tests of the C ABI (no GPU): the library loads, exports every function that
include/flashmask.h declares, and every argument check returns its code before any device work.

Every call below is built to fail a host check, so no kernel is ever launched: pointers are
fake, never dereferenced values."""

import ctypes
import os
import re

import pytest

from mask_aware_flashattention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashmask.h")

FM_OK, FM_ERR_NULL, FM_ERR_SHAPE, FM_ERR_DTYPE, FM_ERR_UNSUPPORTED = 0, 1, 2, 3, 4
FM_ERR_ALIGN, FM_ERR_WORKSPACE, FM_ERR_CHUNKS, FM_ERR_HIP, FM_ERR_VALUE = 5, 6, 7, 8, 9
FM_ERR_SCRATCH = 10

P = ctypes.c_void_p(0x100000)       # fake, 256-byte aligned "device" address (never touched)
P2 = ctypes.c_void_p(0x200000)
MIS = ctypes.c_void_p(0x100002)     # misaligned for tensors (2 bytes)
NUL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from mask_aware_flashattention_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flashmask_\w+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) == 19, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_strerror(lib):
    for s in range(11):
        assert lib.flashmask_strerror(s)
    assert b"unknown" in lib.flashmask_strerror(1234)


def test_tile_sizes(lib):
    v = [ctypes.c_int32() for _ in range(4)]
    refs = [ctypes.byref(x) for x in v]
    assert lib.flashmask_tile_sizes(0, 128, *refs) == FM_OK
    assert [x.value for x in v] == [128, 64, 64, 64]
    assert lib.flashmask_tile_sizes(1, 64, *refs) == FM_OK
    assert lib.flashmask_tile_sizes(0, 64, *refs) == FM_ERR_UNSUPPORTED
    assert lib.flashmask_tile_sizes(1, 128, *refs) == FM_ERR_UNSUPPORTED
    assert lib.flashmask_tile_sizes(7, 128, *refs) == FM_ERR_DTYPE
    assert lib.flashmask_tile_sizes(0, 128, None, *refs[1:]) == FM_ERR_NULL


def shape(B=1, H=2, nq=300, nk=200, d=128, dtype=0):
    return _lib.FmShape(B, H, nq, nk, d, dtype)


def test_workspace_sizes(lib):
    s = shape()
    n_qb, n_kb = 3, 4      # forward tiles 128 x 64
    r = lambda x: -(-x // 256) * 256
    assert lib.flashmask_fwd_workspace_bytes(ctypes.byref(s)) == (
        r(32 * n_kb) + r(4 * n_qb) + r(4 * n_qb * n_kb) + r(4 * n_qb))
    n_qb, n_kb = 5, 4      # dK/dV lists at tiles 64 x 64
    f_qb, f_kb = 3, 4      # dQ lists at the forward tiles 128 x 64
    rows = 1 * 2 * 300
    want = (r(32 * n_kb) + r(4 * n_kb) + r(4 * n_qb * n_kb)
            + r(32 * f_kb) + r(4 * f_qb) + r(4 * f_qb * f_kb)
            + r(4 * n_kb) + r(4 * f_qb) + 2 * r(4 * rows))
    assert lib.flashmask_bwd_workspace_bytes(ctypes.byref(s)) == want
    # the longest square problem: the 64 x 64 grid would hold 2^32 tiles, so the dK/dV lists
    # fall back to 128-key blocks (64 x 128 grid)
    n = 2 ** 22 - 128
    n_qb, n_kb = n // 64, n // 128
    f_qb, f_kb = n // 128, n // 64
    want = (r(32 * n_kb) + r(4 * n_kb) + r(4 * n_qb * n_kb)
            + r(32 * f_kb) + r(4 * f_qb) + r(4 * f_qb * f_kb)
            + r(4 * n_kb) + r(4 * f_qb) + 2 * r(4 * n))
    assert lib.flashmask_bwd_workspace_bytes(ctypes.byref(shape(H=1, nq=n, nk=n))) == want
    assert lib.flashmask_fwd_workspace_bytes(ctypes.byref(shape(d=64))) == 0
    assert lib.flashmask_classify_workspace_bytes(1000, 64) == 512
    assert lib.flashmask_classify_workspace_bytes(0, 64) == 0


def fwd(lib, s, q=P, k=P, v=P, vec=P, o=P2, lse=P2, scale=0.1, ws=P, ws_bytes=0):
    return lib.flashmask_fwd(ctypes.byref(s) if s is not None else None, q, k, v, vec, vec, vec,
                             vec, ctypes.c_float(scale), o, lse, ws, ws_bytes, NUL)


def test_fwd_checks(lib):
    s = shape()
    assert fwd(lib, None) == FM_ERR_NULL
    assert fwd(lib, shape(dtype=5)) == FM_ERR_DTYPE
    assert fwd(lib, shape(d=64)) == FM_ERR_UNSUPPORTED
    assert fwd(lib, shape(dtype=1, d=128)) == FM_ERR_UNSUPPORTED
    for bad in (dict(B=0), dict(H=0), dict(nq=0), dict(nk=0), dict(nq=-5), dict(nk=(1 << 22) + 1)):
        assert fwd(lib, shape(**bad)) == FM_ERR_SHAPE, bad
    assert fwd(lib, s, q=NUL) == FM_ERR_NULL
    assert fwd(lib, s, vec=NUL) == FM_ERR_NULL
    assert fwd(lib, s, lse=NUL) == FM_ERR_NULL
    assert fwd(lib, s, k=MIS) == FM_ERR_ALIGN
    assert fwd(lib, s, vec=ctypes.c_void_p(0x100001)) == FM_ERR_ALIGN
    assert fwd(lib, s, scale=0.0) == FM_ERR_VALUE
    assert fwd(lib, s, scale=-1.0) == FM_ERR_VALUE
    assert fwd(lib, s, scale=float("nan")) == FM_ERR_VALUE
    assert fwd(lib, s, scale=float("inf")) == FM_ERR_VALUE
    need = lib.flashmask_fwd_workspace_bytes(ctypes.byref(s))
    assert fwd(lib, s, ws_bytes=need - 1) == FM_ERR_WORKSPACE
    assert fwd(lib, s, ws=NUL, ws_bytes=need) == FM_ERR_WORKSPACE


def bwd(lib, s, ptrs=None, scale=0.1, ws=P, ws_bytes=0):
    p = dict(q=P, k=P, v=P, o=P, do=P, lse=P2, vec=P, dq=P2, dk=P2, dv=P2)
    p.update(ptrs or {})
    return lib.flashmask_bwd(ctypes.byref(s), p["q"], p["k"], p["v"], p["o"], p["do"], p["lse"],
                             p["vec"], p["vec"], p["vec"], p["vec"], ctypes.c_float(scale),
                             p["dq"], p["dk"], p["dv"], ws, ws_bytes, NUL)


def test_bwd_checks(lib):
    s = shape()
    for name in ("q", "k", "v", "o", "do", "lse", "vec", "dq", "dk", "dv"):
        assert bwd(lib, s, {name: NUL}) == FM_ERR_NULL, name
    for name in ("q", "k", "v", "o", "do", "dq", "dk", "dv"):
        assert bwd(lib, s, {name: MIS}) == FM_ERR_ALIGN, name
    assert bwd(lib, shape(nq=0)) == FM_ERR_SHAPE
    assert bwd(lib, s, scale=0.0) == FM_ERR_VALUE
    need = lib.flashmask_bwd_workspace_bytes(ctypes.byref(s))
    assert bwd(lib, s, ws_bytes=need - 1) == FM_ERR_WORKSPACE


def localize(lib, starts, lens, n=0, nq_global=100, vec=P, n_local=None):
    out = n_local if n_local is not None else ctypes.c_int32(-1)
    a = (ctypes.c_int32 * max(len(starts), 1))(*starts)
    b = (ctypes.c_int32 * max(len(lens), 1))(*lens)
    st = lib.flashmask_localize(vec, vec, vec, vec, n, nq_global, a, b, len(starts), P2, P2, P2,
                                P2, ctypes.byref(out), NUL)
    return st, out.value


def test_localize_chunk_checks(lib):
    assert localize(lib, [10, 50], [20, 30]) == (FM_OK, 50)       # n = 0: no device work
    assert localize(lib, [0], [100]) == (FM_OK, 100)
    assert localize(lib, [50, 10], [5, 5])[0] == FM_ERR_CHUNKS     # unsorted
    assert localize(lib, [10, 12], [5, 5])[0] == FM_ERR_CHUNKS     # overlapping
    assert localize(lib, [10], [0])[0] == FM_ERR_CHUNKS            # empty chunk
    assert localize(lib, [-1], [5])[0] == FM_ERR_CHUNKS            # negative offset
    assert localize(lib, [98], [5])[0] == FM_ERR_CHUNKS            # past nq_global
    assert localize(lib, [], [])[0] == FM_ERR_CHUNKS               # no chunk
    assert localize(lib, list(range(0, 130, 2)), [1] * 65, nq_global=200)[0] == FM_ERR_CHUNKS
    assert localize(lib, list(range(0, 128, 2)), [1] * 64, nq_global=200) == (FM_OK, 64)
    assert localize(lib, [0], [5], n=-1)[0] == FM_ERR_SHAPE
    assert localize(lib, [0], [5], n=10, vec=NUL)[0] == FM_ERR_NULL
    assert localize(lib, [0], [5], n=10, vec=ctypes.c_void_p(0x100001))[0] == FM_ERR_ALIGN
    st = lib.flashmask_localize(P, P, P, P, 0, 10, (ctypes.c_int32 * 1)(0), (ctypes.c_int32 * 1)(5),
                                1, P2, P2, P2, P2, None, NUL)
    assert st == FM_ERR_NULL


def test_classify_checks(lib):
    def call(vec=P, nq=100, nk=100, BM=16, BN=16, kcnt=P2, klist=P2, ws=P, ws_bytes=0):
        return lib.flashmask_classify(vec, vec, vec, vec, nq, nk, BM, BN, P2, P2, P2, kcnt, klist,
                                      ws, ws_bytes, NUL)
    assert call(vec=NUL) == FM_ERR_NULL
    assert call(nq=0) == FM_ERR_SHAPE
    assert call(BN=0) == FM_ERR_SHAPE
    assert call(BM=-1) == FM_ERR_SHAPE
    assert call(nq=1 << 30, nk=1 << 30, BM=1, BN=1) == FM_ERR_SHAPE
    assert call(kcnt=NUL) == FM_ERR_NULL          # kcnt and klist go together
    assert call(ws_bytes=10) == FM_ERR_WORKSPACE
    assert call(ws=NUL, ws_bytes=1 << 20) == FM_ERR_WORKSPACE


def test_block_order_checks(lib):
    assert lib.flashmask_block_order(NUL, 4, P2, NUL) == FM_ERR_NULL
    assert lib.flashmask_block_order(P2, 4, NUL, NUL) == FM_ERR_NULL
    assert lib.flashmask_block_order(P2, 0, P2, NUL) == FM_ERR_SHAPE
    assert lib.flashmask_block_order(ctypes.c_void_p(0x100002), 4, P2, NUL) == FM_ERR_ALIGN


def test_prune_checks(lib):
    assert lib.flashmask_prune_workspace_bytes(1000, 300, 100, 64) == 512 + 256  # 16 chunks, 3 blocks
    assert lib.flashmask_prune_workspace_bytes(0, 300, 100, 64) == 0

    def call(vec=P, live=P2, nk=1000, n_local=300, BM=100, chunk=64, ws=P, ws_bytes=1 << 20):
        return lib.flashmask_prune_chunks(vec, vec, vec, vec, nk, n_local, BM, chunk, live, ws,
                                          ws_bytes, NUL)
    assert call(vec=NUL) == FM_ERR_NULL
    assert call(live=NUL) == FM_ERR_NULL
    for bad in (dict(nk=0), dict(n_local=0), dict(BM=0), dict(chunk=-3)):
        assert call(**bad) == FM_ERR_SHAPE, bad
    assert call(live=ctypes.c_void_p(0x200002)) == FM_ERR_ALIGN
    assert call(ws_bytes=767) == FM_ERR_WORKSPACE
    assert call(ws=NUL) == FM_ERR_WORKSPACE


def layout(B=1, H=2, H_kv=None, nq=300, nk=200, d=128, dtype=0, mask_b=1, mask_h=1, qs=None,
           ks=None):
    l = _lib.FmLayout()
    l.B, l.H, l.H_kv, l.nq, l.nk, l.d, l.dtype = B, H, H if H_kv is None else H_kv, nq, nk, d, dtype
    l.mask_b, l.mask_h = mask_b, mask_h
    hk = l.H_kv
    for i, x in enumerate(qs or (H * nq * d, nq * d, d)):
        l.q_stride[i] = x
    for i, x in enumerate(ks or (hk * nk * d, nk * d, d)):
        l.kv_stride[i] = x
    return l


def test_ex_workspace_matches_plain_and_scales_with_mask_sets(lib):
    r = lambda x: -(-x // 256) * 256
    assert (lib.flashmask_fwd_ex_workspace_bytes(ctypes.byref(layout()))
            == lib.flashmask_fwd_workspace_bytes(ctypes.byref(shape())))
    assert (lib.flashmask_bwd_ex_workspace_bytes(ctypes.byref(layout()))
            == lib.flashmask_bwd_workspace_bytes(ctypes.byref(shape())))
    n_qb, n_kb, sets = 3, 4, 2 * 2   # mask per batch and head, B = H = 2
    l = layout(B=2, mask_b=2, mask_h=2)
    assert lib.flashmask_fwd_ex_workspace_bytes(ctypes.byref(l)) == (
        r(32 * n_kb * sets) + r(4 * n_qb * sets) + r(4 * n_qb * n_kb * sets) + r(4 * n_qb * sets))
    n_qb, n_kb = 5, 4
    f_qb, f_kb = 3, 4
    rows = 2 * 2 * 300
    want = (r(32 * n_kb * sets) + r(4 * n_kb * sets) + r(4 * n_qb * n_kb * sets)
            + r(32 * f_kb * sets) + r(4 * f_qb * sets) + r(4 * f_qb * f_kb * sets)
            + r(4 * n_kb * sets) + r(4 * f_qb * sets) + 2 * r(4 * rows))
    assert lib.flashmask_bwd_ex_workspace_bytes(ctypes.byref(l)) == want
    assert lib.flashmask_fwd_ex_workspace_bytes(None) == 0


def fwd_ex(lib, l, q=P, vec=P, scale=0.1, ws=P, ws_bytes=0):
    return lib.flashmask_fwd_ex(ctypes.byref(l) if l is not None else None, q, P, P, vec, vec, vec,
                                vec, ctypes.c_float(scale), P2, P2, ws, ws_bytes, NUL)


def bwd_ex(lib, l, dk=P2, scale=0.1, ws_bytes=0):
    return lib.flashmask_bwd_ex(ctypes.byref(l), P, P, P, P, P, P2, P, P, P, P,
                                ctypes.c_float(scale), P2, dk, P2, P, ws_bytes, NUL)


def test_ex_layout_checks(lib):
    assert fwd_ex(lib, None) == FM_ERR_NULL
    assert fwd_ex(lib, layout(dtype=4)) == FM_ERR_DTYPE
    assert fwd_ex(lib, layout(d=64)) == FM_ERR_UNSUPPORTED
    assert fwd_ex(lib, layout()) == FM_ERR_WORKSPACE          # everything else valid
    assert fwd_ex(lib, layout(H=4, H_kv=2)) == FM_ERR_WORKSPACE
    assert fwd_ex(lib, layout(B=2, H=4, mask_b=2, mask_h=4)) == FM_ERR_WORKSPACE
    shape_errors = [
        dict(H=4, H_kv=3),                    # H_kv does not divide H
        dict(H_kv=0),
        dict(B=2, mask_b=3),                  # mask sets: 1 or B, 1 or H
        dict(mask_h=3),
        dict(qs=(2 * 300 * 128, 300 * 128, 120)),   # row stride below d
        dict(ks=(-8, 200 * 128, 128)),               # negative stride
        dict(nk=200, ks=(0, 0, 1 << 25)),            # K rows span 4 GiB or more
        dict(nq=0),
        dict(nk=(1 << 22) + 1),
    ]
    for kw in shape_errors:
        assert fwd_ex(lib, layout(**kw)) == FM_ERR_SHAPE, kw
    # outputs are written through the same strides: no two (batch, head, row) may share memory
    overlap = [
        dict(H=2, qs=(2 * 300 * 128, 0, 128)),            # zero head stride, two heads
        dict(B=2, qs=(0, 300 * 128, 128)),                # zero batch stride, two batches
        dict(H=2, qs=(2 * 300 * 128, 128 * 100, 128)),    # head 1 starts inside head 0's rows
        dict(H=2, H_kv=2, ks=(2 * 200 * 128, 64, 256)),   # heads interleave with a half row
    ]
    for kw in overlap:
        assert fwd_ex(lib, layout(**kw)) == FM_ERR_SHAPE, kw
        assert bwd_ex(lib, layout(**kw)) == FM_ERR_SHAPE, kw
    # packed [B, n, 3, H, d] projections: heads interleave inside a row without overlapping
    assert fwd_ex(lib, layout(B=2, H=4, qs=(300 * 3 * 4 * 128, 128, 3 * 4 * 128),
                              ks=(200 * 3 * 4 * 128, 128, 3 * 4 * 128))) == FM_ERR_WORKSPACE
    # the rows of the ragged last 128-row tile are addressed too: nq = 1365 rows of 3 MiB end
    # below 4 GiB, but 1408 (the next multiple of 128) do not
    wide = 3 * (1 << 19)
    assert fwd_ex(lib, layout(H=1, nq=1365, qs=(1365 * wide, 1365 * wide, wide))) == FM_ERR_SHAPE
    assert fwd_ex(lib, layout(H=1, nq=1280, qs=(1280 * wide, 1280 * wide, wide))) == FM_ERR_WORKSPACE
    # every row start 16-byte aligned: strides * 2 bytes must be multiples of 16
    assert fwd_ex(lib, layout(qs=(2 * 300 * 128, 300 * 128 + 4, 128))) == FM_ERR_ALIGN
    assert fwd_ex(lib, layout(ks=(2 * 200 * 128, 200 * 128, 132))) == FM_ERR_ALIGN
    assert fwd_ex(lib, layout(), q=NUL) == FM_ERR_NULL
    assert fwd_ex(lib, layout(), q=MIS) == FM_ERR_ALIGN
    assert fwd_ex(lib, layout(), vec=NUL) == FM_ERR_NULL
    assert fwd_ex(lib, layout(), scale=float("nan")) == FM_ERR_VALUE
    need = lib.flashmask_fwd_ex_workspace_bytes(ctypes.byref(layout()))
    assert fwd_ex(lib, layout(), ws_bytes=need - 1) == FM_ERR_WORKSPACE
    assert fwd_ex(lib, layout(), ws=NUL, ws_bytes=need) == FM_ERR_WORKSPACE


def test_bwd_ex_checks(lib):
    assert bwd_ex(lib, layout()) == FM_ERR_WORKSPACE
    assert bwd_ex(lib, layout(H=4, H_kv=1)) == FM_ERR_WORKSPACE
    assert bwd_ex(lib, layout(H=512, H_kv=1, nq=128, nk=128)) == FM_ERR_SHAPE  # group above 256
    # the dK/dV kernel spans a group's query heads: (G-1) head strides + the rows < 4 GiB
    assert fwd_ex(lib, layout(H=4, H_kv=1, qs=(0, 1 << 30, 128))) == FM_ERR_WORKSPACE
    assert bwd_ex(lib, layout(H=4, H_kv=1, qs=(0, 1 << 30, 128))) == FM_ERR_SHAPE
    assert bwd_ex(lib, layout(), dk=NUL) == FM_ERR_NULL
    assert bwd_ex(lib, layout(), dk=MIS) == FM_ERR_ALIGN
    assert bwd_ex(lib, layout(), scale=0.0) == FM_ERR_VALUE


def test_noalloc_checks(lib):
    """The no-alloc forward refuses a problem larger than its fixed array, and otherwise runs
    the forward's own argument checks, all before any device work."""
    assert lib.flashmask_fwd_noalloc_max_workspace_bytes() == 16 << 20

    def call(s, q=P, scale=0.1):
        return lib.flashmask_fwd_noalloc(ctypes.byref(s) if s is not None else None, q, P, P, P,
                                         P, P, P, ctypes.c_float(scale), P2, P2, NUL)
    assert call(None) == FM_ERR_NULL
    assert call(shape(nq=1 << 18, nk=1 << 18, H=1)) == FM_ERR_SCRATCH   # 32 MiB of lists
    assert call(shape(d=64)) == FM_ERR_UNSUPPORTED
    assert call(shape(nq=0)) == FM_ERR_SHAPE
    assert call(shape(), q=NUL) == FM_ERR_NULL   # before the device is touched


def test_debug_library_exports_the_stamp_calls_and_the_abi():
    """The timeline build (libflashmask_stamps.so) exports everything include/flashmask.h
    declares plus the three calls of include/flashmask_debug.h, which the default library
    lacks; a null or oversized copy request is refused before any device work."""
    from mask_aware_flashattention_amd import build
    from mask_aware_flashattention_amd.wg_timeline import LIB_STAMPS
    if not os.path.exists(LIB_STAMPS):
        build.build(stamps=True)
    dbg = ctypes.CDLL(LIB_STAMPS)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "flashmask_debug.h")).read(),
                  flags=re.S)
    debug_names = sorted(set(re.findall(r"\b(flashmask_\w+)\s*\(", text)))
    assert debug_names == ["flashmask_debug_stamps_dkdv", "flashmask_debug_stamps_dq",
                           "flashmask_debug_stamps_fwd"]
    for n in declared_functions() + debug_names:
        assert hasattr(dbg, n), n
    plain = ctypes.CDLL(_lib.LIB_PATH)
    for n in debug_names:
        assert not hasattr(plain, n), n
        f = getattr(dbg, n)
        f.restype, f.argtypes = ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t]
        assert f(None, 8) == -1
        assert f(ctypes.c_void_p(0x1000), (1 << 16) * 8 * 8 + 8) == -1
