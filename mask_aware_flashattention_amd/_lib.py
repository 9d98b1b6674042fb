"""ctypes loader for ``libflashmask.so`` (built in-tree by ``mask_aware_flashattention_amd.build``).

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing, loading raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflashmask.so")

FM_OK = 0
FM_BF16 = 0
FM_FP32 = 1

c_i32 = ctypes.c_int32
c_p = ctypes.c_void_p
c_i32p = ctypes.POINTER(ctypes.c_int32)


class FmShape(ctypes.Structure):
    _fields_ = [("B", c_i32), ("H", c_i32), ("nq", c_i32), ("nk", c_i32), ("d", c_i32),
                ("dtype", c_i32)]


class FmLayout(ctypes.Structure):
    _fields_ = [("B", c_i32), ("H", c_i32), ("H_kv", c_i32), ("nq", c_i32), ("nk", c_i32),
                ("d", c_i32), ("dtype", c_i32), ("mask_b", c_i32), ("mask_h", c_i32),
                ("q_stride", ctypes.c_int64 * 3), ("kv_stride", ctypes.c_int64 * 3)]


# name -> (restype, argtypes)
SIGNATURES = {
    "flashmask_strerror": (ctypes.c_char_p, [c_i32]),
    "flashmask_tile_sizes": (c_i32, [c_i32, c_i32, c_i32p, c_i32p, c_i32p, c_i32p]),
    "flashmask_fwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(FmShape)]),
    "flashmask_fwd": (c_i32, [ctypes.POINTER(FmShape), c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                              ctypes.c_float, c_p, c_p, c_p, ctypes.c_size_t, c_p]),
    "flashmask_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(FmShape)]),
    "flashmask_bwd": (c_i32, [ctypes.POINTER(FmShape), c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                              c_p, c_p, ctypes.c_float, c_p, c_p, c_p, c_p, ctypes.c_size_t, c_p]),
    "flashmask_localize": (c_i32, [c_p, c_p, c_p, c_p, c_i32, c_i32, c_i32p, c_i32p, c_i32,
                                   c_p, c_p, c_p, c_p, c_i32p, c_p]),
    "flashmask_classify_workspace_bytes": (ctypes.c_size_t, [c_i32, c_i32]),
    "flashmask_set_profile_events": (c_i32, [c_p, c_p, c_p, c_p]),
    "flashmask_block_order": (c_i32, [c_p, c_i32, c_p, c_p]),
    "flashmask_prune_workspace_bytes": (ctypes.c_size_t, [c_i32, c_i32, c_i32, c_i32]),
    "flashmask_prune_chunks": (c_i32, [c_p, c_p, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_p, c_p,
                                       ctypes.c_size_t, c_p]),
    "flashmask_classify": (c_i32, [c_p, c_p, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_p, c_p,
                                   c_p, c_p, c_p, c_p, ctypes.c_size_t, c_p]),
    "flashmask_fwd_ex_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(FmLayout)]),
    "flashmask_fwd_ex": (c_i32, [ctypes.POINTER(FmLayout), c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                                 ctypes.c_float, c_p, c_p, c_p, ctypes.c_size_t, c_p]),
    "flashmask_fwd_noalloc_max_workspace_bytes": (ctypes.c_size_t, []),
    "flashmask_fwd_noalloc": (c_i32, [ctypes.POINTER(FmShape), c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                                      ctypes.c_float, c_p, c_p, c_p]),
    "flashmask_bwd_ex_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(FmLayout)]),
    "flashmask_bwd_ex": (c_i32, [ctypes.POINTER(FmLayout), c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                                 c_p, c_p, c_p, ctypes.c_float, c_p, c_p, c_p, c_p,
                                 ctypes.c_size_t, c_p]),
}

_lib = None


class FlashMaskError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def load(path: str = LIB_PATH):
    """Load the library once; raises RuntimeError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m mask_aware_flashattention_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().flashmask_strerror(status).decode()


def check(status: int, where: str):
    if status != FM_OK:
        raise FlashMaskError(status, where)
