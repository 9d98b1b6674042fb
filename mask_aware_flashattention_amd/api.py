"""Python binding of the C ABI on torch tensors.

PyTorch provides device memory and the current stream; the tensors' pointers go straight to
``libflashmask.so``.  No computation happens here.
"""

from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import FmLayout, FmShape, check

_DTYPES = {torch.bfloat16: _lib.FM_BF16, torch.float32: _lib.FM_FP32}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_cuda(*ts):
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a ROCm/CUDA device")
        if t.device != dev:
            raise ValueError("tensors must be on one device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _vectors(lts, lte, uts, ute, nk):
    for v in (lts, lte, uts, ute):
        if v.dtype != torch.int32 or v.dim() != 1 or v.numel() != nk:
            raise ValueError(f"mask vectors must be int32 [{nk}]")
    _require_cuda(lts, lte, uts, ute)


def _expect(t, name, shape, dtype):
    """t must have exactly this shape and dtype (checked before any pointer is passed on: the C
    interface sees no tensor sizes, so a short or mistyped buffer would be read or written out
    of bounds)."""
    if t is None:
        raise ValueError(f"{name} is missing")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _shape(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B, H, nq, d] and k, v [B, H, nk, d]")
    B, H, nq, d = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError("q and k disagree on B, H or d")
    if q.dtype not in _DTYPES:
        raise ValueError("dtype must be bfloat16 or float32")
    _expect(k, "k", k.shape, q.dtype)
    _expect(v, "v", k.shape, q.dtype)
    return FmShape(B, H, nq, k.shape[2], d, _DTYPES[q.dtype])


def _check_workspace(ws, device):
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    if ws.device != device:
        raise ValueError("workspace must be on the tensors' device")


def tile_sizes(dtype=torch.bfloat16, d: int = 128):
    lib = _lib.load()
    out = [ctypes.c_int32() for _ in range(4)]
    check(lib.flashmask_tile_sizes(_DTYPES[dtype], d, *[ctypes.byref(x) for x in out]),
          "flashmask_tile_sizes")
    return tuple(x.value for x in out)


def fwd_workspace_bytes(shape: FmShape) -> int:
    return _lib.load().flashmask_fwd_workspace_bytes(ctypes.byref(shape))


def bwd_workspace_bytes(shape: FmShape) -> int:
    return _lib.load().flashmask_bwd_workspace_bytes(ctypes.byref(shape))


def _workspace(nbytes, device):
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def fwd(q, k, v, lts, lte, uts, ute, scale=None, *, out=None, lse=None, workspace=None):
    """O, LSE = masked attention forward.  q [B,H,nq,d], k/v [B,H,nk,d] (bf16 d=128 or fp32
    d=64), mask vectors int32 [nk].  Returns (O like q, LSE float32 [B,H,nq])."""
    lib = _lib.load()
    shape = _shape(q, k, v)
    if out is not None:
        _expect(out, "out", q.shape, q.dtype)
    if lse is not None:
        _expect(lse, "lse", q.shape[:3], torch.float32)
    _require_cuda(q, k, v, *[t for t in (out, lse) if t is not None])
    _vectors(lts, lte, uts, ute, shape.nk)
    if scale is None:
        scale = 1.0 / math.sqrt(shape.d)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse is None else lse
    ws = workspace if workspace is not None else _workspace(fwd_workspace_bytes(shape), q.device)
    _check_workspace(ws, q.device)
    st = lib.flashmask_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(lts), _ptr(lte),
                           _ptr(uts), _ptr(ute), ctypes.c_float(scale), _ptr(o), _ptr(lse_t),
                           _ptr(ws), ws.numel(), _stream(q.device))
    check(st, "flashmask_fwd")
    return o, lse_t


def fwd_noalloc(q, k, v, lts, lte, uts, ute, scale=None, *, out, lse):
    """The forward without a workspace (flashmask_fwd_noalloc): the library's fixed 16 MiB
    device array stands in for it, so nothing is allocated here either; out and lse must be
    given.  Calls that overlap in time on one GPU race on that array."""
    lib = _lib.load()
    shape = _shape(q, k, v)
    _expect(out, "out", q.shape, q.dtype)
    _expect(lse, "lse", q.shape[:3], torch.float32)
    _require_cuda(q, k, v, out, lse)
    _vectors(lts, lte, uts, ute, shape.nk)
    if scale is None:
        scale = 1.0 / math.sqrt(shape.d)
    st = lib.flashmask_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(lts),
                                   _ptr(lte), _ptr(uts), _ptr(ute), ctypes.c_float(scale),
                                   _ptr(out), _ptr(lse), _stream(q.device))
    check(st, "flashmask_fwd_noalloc")
    return out, lse


def bwd(q, k, v, o, do, lse, lts, lte, uts, ute, scale=None, *, workspace=None, grads=None):
    """dQ, dK, dV of L = sum(O * dO).  ``o`` and ``lse`` are the forward's outputs."""
    lib = _lib.load()
    shape = _shape(q, k, v)
    _expect(o, "o", q.shape, q.dtype)
    _expect(do, "do", q.shape, q.dtype)
    _expect(lse, "lse", q.shape[:3], torch.float32)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = grads
        _expect(dq, "dq", q.shape, q.dtype)
        _expect(dk, "dk", k.shape, q.dtype)
        _expect(dv, "dv", k.shape, q.dtype)
    _require_cuda(q, k, v, o, do, lse, dq, dk, dv)
    _vectors(lts, lte, uts, ute, shape.nk)
    if scale is None:
        scale = 1.0 / math.sqrt(shape.d)
    ws = workspace if workspace is not None else _workspace(bwd_workspace_bytes(shape), q.device)
    _check_workspace(ws, q.device)
    st = lib.flashmask_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                           _ptr(lse), _ptr(lts), _ptr(lte), _ptr(uts), _ptr(ute),
                           ctypes.c_float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                           ws.numel(), _stream(q.device))
    check(st, "flashmask_bwd")
    return dq, dk, dv


def _layout(q, k, v, vec):
    """fm_layout of strided q [B,H,nq,d] and k, v [B,H_kv,nk,d] views and mask vectors of shape
    [nk] (shared), [H, nk] (per head) or [mask_b, mask_h, nk] with mask_b in {1, B} and mask_h
    in {1, H}."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B, H, nq, d] and k, v [B, H_kv, nk, d]")
    B, H, nq, d = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d or v.shape != k.shape or v.stride() != k.stride():
        raise ValueError("k and v must have equal shapes [B, H_kv, nk, d] and equal strides")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("dtype must be bfloat16 or float32, the same for q, k, v")
    if q.stride(3) != 1 or k.stride(3) != 1:
        raise ValueError("the d axis must be contiguous")
    _no_overlap(q, "q")
    _no_overlap(k, "k")
    if q.device != k.device or q.device != v.device or not q.is_cuda:
        raise ValueError("q, k, v must be on one ROCm/CUDA device")
    if vec.dim() == 1:
        mb, mh = 1, 1
    elif vec.dim() == 2:
        mb, mh = 1, vec.shape[0]
    elif vec.dim() == 3:
        mb, mh = vec.shape[0], vec.shape[1]
    else:
        raise ValueError("mask vectors must be [nk], [H, nk] or [mask_b, mask_h, nk]")
    lay = FmLayout()
    lay.B, lay.H, lay.H_kv, lay.nq, lay.nk, lay.d = B, H, Hkv, nq, nk, d
    lay.dtype, lay.mask_b, lay.mask_h = _DTYPES[q.dtype], mb, mh
    for i in range(3):
        lay.q_stride[i] = q.stride(i)
        lay.kv_stride[i] = k.stride(i)
    return lay


def _no_overlap(t, name):
    """No two (batch, head, row) positions of t's layout may share memory: outputs are created
    with (and written through) the same strides, so a zero batch or head stride (an expanded
    view) or interleaved heads would make workgroups write the same bytes."""
    B, H, n, d = t.shape
    span = d
    for extent, stride in sorted(((B, t.stride(0)), (H, t.stride(1)), (n, t.stride(2))),
                                 key=lambda x: x[1]):
        if extent <= 1:
            continue
        if stride < span:
            raise ValueError(f"{name}: batch, head and row strides {t.stride()[:3]} overlap "
                             f"(an expanded or interleaved view); pass a copy")
        span = (extent - 1) * stride + span


def _vector_sets(lts, lte, uts, ute, nk):
    for x in (lts, lte, uts, ute):
        if x.dtype != torch.int32 or x.shape[-1] != nk or x.shape != lts.shape:
            raise ValueError(f"mask vectors must be int32 [..., {nk}] of one shape")
        if not x.is_cuda or not x.is_contiguous():
            raise ValueError("mask vectors must be contiguous device tensors")


def _like_strided(t, like):
    """Empty tensor with like's shape and strides (the layout the extended calls require)."""
    return torch.empty_strided(like.shape, like.stride(), dtype=like.dtype, device=like.device)


def fwd_ex(q, k, v, lts, lte, uts, ute, scale=None, *, out=None, lse=None, workspace=None):
    """Forward on strided views: q [B,H,nq,d], k/v [B,H_kv,nk,d] (H_kv divides H: grouped
    heads), mask vectors [nk], [H, nk] or [mask_b, mask_h, nk].  O has q's strides; LSE is
    contiguous float32 [B,H,nq]."""
    lib = _lib.load()
    lay = _layout(q, k, v, lts)
    _vector_sets(lts, lte, uts, ute, lay.nk)
    if scale is None:
        scale = 1.0 / math.sqrt(lay.d)
    o = _like_strided(None, q) if out is None else out
    _expect(o, "out", q.shape, q.dtype)
    if o.stride() != q.stride() or o.device != q.device:
        raise ValueError("out must have q's strides and device")
    if lse is not None:
        _expect(lse, "lse", q.shape[:3], torch.float32)
        _require_cuda(lse)
        if lse.device != q.device:
            raise ValueError("lse must be on q's device")
    lse_t = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse is None else lse
    nbytes = lib.flashmask_fwd_ex_workspace_bytes(ctypes.byref(lay))
    ws = workspace if workspace is not None else _workspace(nbytes, q.device)
    _check_workspace(ws, q.device)
    st = lib.flashmask_fwd_ex(ctypes.byref(lay), _ptr(q), _ptr(k), _ptr(v), _ptr(lts), _ptr(lte),
                              _ptr(uts), _ptr(ute), ctypes.c_float(scale), _ptr(o), _ptr(lse_t),
                              _ptr(ws), ws.numel(), _stream(q.device))
    check(st, "flashmask_fwd_ex")
    return o, lse_t


def bwd_ex(q, k, v, o, do, lse, lts, lte, uts, ute, scale=None, *, workspace=None):
    """dQ, dK, dV on strided views (see fwd_ex); o, do and dQ share q's strides, dK and dV k's.
    With grouped heads dK and dV of a key/value head sum over its query heads."""
    lib = _lib.load()
    lay = _layout(q, k, v, lts)
    _vector_sets(lts, lte, uts, ute, lay.nk)
    _expect(o, "o", q.shape, q.dtype)
    _expect(do, "do", q.shape, q.dtype)
    _expect(lse, "lse", q.shape[:3], torch.float32)
    if o.stride() != q.stride() or do.stride() != q.stride():
        raise ValueError("o and do must have q's strides")
    _require_cuda(lse)
    if o.device != q.device or do.device != q.device or lse.device != q.device:
        raise ValueError("o, do and lse must be on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(lay.d)
    dq, dk, dv = _like_strided(None, q), _like_strided(None, k), _like_strided(None, v)
    nbytes = lib.flashmask_bwd_ex_workspace_bytes(ctypes.byref(lay))
    ws = workspace if workspace is not None else _workspace(nbytes, q.device)
    _check_workspace(ws, q.device)
    st = lib.flashmask_bwd_ex(ctypes.byref(lay), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                              _ptr(lse), _ptr(lts), _ptr(lte), _ptr(uts), _ptr(ute),
                              ctypes.c_float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                              ws.numel(), _stream(q.device))
    check(st, "flashmask_bwd_ex")
    return dq, dk, dv


def localize(lts, lte, uts, ute, chunk_start, chunk_len, nq_global):
    """Rank-local vectors by clip-shift-max for the rank owning the given query-row chunks."""
    lib = _lib.load()
    n = lts.numel()
    _vectors(lts, lte, uts, ute, n)
    starts = (ctypes.c_int32 * len(chunk_start))(*[int(x) for x in chunk_start])
    lens = (ctypes.c_int32 * len(chunk_len))(*[int(x) for x in chunk_len])
    if len(chunk_start) != len(chunk_len):
        raise ValueError("chunk_start and chunk_len differ in length")
    outs = [torch.empty_like(x) for x in (lts, lte, uts, ute)]
    n_local = ctypes.c_int32()
    st = lib.flashmask_localize(_ptr(lts), _ptr(lte), _ptr(uts), _ptr(ute), n, int(nq_global),
                                starts, lens, len(chunk_start), *[_ptr(x) for x in outs],
                                ctypes.byref(n_local), _stream(lts.device))
    check(st, "flashmask_localize")
    return (*outs, n_local.value)


def classify(lts, lte, uts, ute, nq, BM, BN, *, cls=True, qlists=True, klists=True):
    """Tile classes and compacted lists at tile shape (BM, BN); returns a dict of tensors
    (cls uint8 [n_qb, n_kb], qcnt, qlist [n_qb, n_kb], kcnt, klist [n_kb, n_qb])."""
    lib = _lib.load()
    nk = lts.numel()
    _vectors(lts, lte, uts, ute, nk)
    dev = lts.device
    n_qb, n_kb = -(-nq // BM), -(-nk // BN)
    out = {}
    if cls:
        out["cls"] = torch.empty((n_qb, n_kb), dtype=torch.uint8, device=dev)
    if qlists:
        out["qcnt"] = torch.empty(n_qb, dtype=torch.int32, device=dev)
        out["qlist"] = torch.empty((n_qb, n_kb), dtype=torch.int32, device=dev)
    if klists:
        out["kcnt"] = torch.empty(n_kb, dtype=torch.int32, device=dev)
        out["klist"] = torch.empty((n_kb, n_qb), dtype=torch.int32, device=dev)
    ws = _workspace(lib.flashmask_classify_workspace_bytes(nk, BN), dev)
    st = lib.flashmask_classify(_ptr(lts), _ptr(lte), _ptr(uts), _ptr(ute), nq, nk, BM, BN,
                                _ptr(out.get("cls")), _ptr(out.get("qcnt")),
                                _ptr(out.get("qlist")), _ptr(out.get("kcnt")),
                                _ptr(out.get("klist")), _ptr(ws), ws.numel(), _stream(dev))
    check(st, "flashmask_classify")
    return out


def block_order(cnt):
    """Work order of the attention kernels for block counts `cnt` (int32 device tensor): four
    buckets by count, largest first, descending index inside a bucket; returns an int32
    permutation tensor."""
    lib = _lib.load()
    if cnt.dtype != torch.int32 or not cnt.is_contiguous():
        raise ValueError("cnt must be a contiguous int32 tensor")
    order = torch.empty_like(cnt)
    check(lib.flashmask_block_order(_ptr(cnt), cnt.numel(), _ptr(order), _stream(cnt.device)),
          "flashmask_block_order")
    return order


def prune_chunks(lts, lte, uts, ute, n_local, BM, chunk):
    """Per key chunk of `chunk` keys, the number of BM-row blocks of the rank's n_local rows whose
    tile is not fully masked (0: the rank never needs the chunk), from localised vectors."""
    lib = _lib.load()
    nk = lts.numel()
    _vectors(lts, lte, uts, ute, nk)
    dev = lts.device
    live = torch.empty(-(-nk // chunk), dtype=torch.int32, device=dev)
    ws = _workspace(lib.flashmask_prune_workspace_bytes(nk, n_local, BM, chunk), dev)
    check(lib.flashmask_prune_chunks(_ptr(lts), _ptr(lte), _ptr(uts), _ptr(ute), nk, int(n_local),
                                     int(BM), int(chunk), _ptr(live), _ptr(ws), ws.numel(),
                                     _stream(dev)), "flashmask_prune_chunks")
    return live
