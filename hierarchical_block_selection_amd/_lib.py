"""ctypes declarations of libpisa's C ABI (include/pisa.h)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpisa.so")

PISA_OK = 0
PISA_ERR_INVALID = -1
PISA_ERR_UNSUPPORTED = -2
PISA_ERR_WORKSPACE = -3
PISA_ERR_HIP = -4

PISA_F32 = 0
PISA_BF16 = 1
PISA_CAUSAL = 1
PISA_FORCE_FIRST_PREV = 2
PISA_SCORE_MEAN = 4
PISA_SCORE_MEAN_VAR = 8
PISA_MAX_LEVELS = 32
PISA_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

PISA_OP_PYRAMID, PISA_OP_SELECT, PISA_OP_BSA, PISA_OP_ATTN, PISA_OP_DECODE, PISA_OP_ATTN_BWD = range(6)
PISA_SELECT_AUTO, PISA_SELECT_FUSED, PISA_SELECT_TWO_STAGE = range(3)

EXPORTED = (
    "pisa_pyramid_layout", "pisa_workspace_bytes", "pisa_build_pyramid", "pisa_select",
    "pisa_select_noalloc", "pisa_bsa_select", "pisa_block_sparse_attn", "pisa_block_sparse_attn_backward",
    "pisa_pyramid_append", "pisa_decode_step",
    "pisa_status_string",
    "pisa_last_error", "pisa_profile_enable", "pisa_profile_report",
)


class PisaProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("branch", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
    ]


class PisaError(RuntimeError):
    def __init__(self, func, status, detail):
        super().__init__(f"{func} failed with status {status}: {detail}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libpisa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m hierarchical_block_selection_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pp = ctypes.POINTER(PisaProblem)
    i32 = ctypes.c_int32
    sig = {
        "pisa_pyramid_layout": [i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_int64), i32],
        "pisa_workspace_bytes": [pp, i32, ctypes.POINTER(sz)],
        "pisa_build_pyramid": [pp, vp, vp, vp],
        "pisa_pyramid_append": [pp, vp, vp, vp, vp],
        "pisa_select": [pp, vp, vp, vp, vp, vp, i32, vp, sz, vp],
        "pisa_select_noalloc": [pp, vp, vp, vp, vp, vp, i32, vp],
        "pisa_bsa_select": [pp, vp, vp, vp, vp, vp, sz, vp],
        "pisa_block_sparse_attn": [pp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "pisa_block_sparse_attn_backward": [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "pisa_decode_step": [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.pisa_profile_enable.argtypes = [ctypes.c_int]
    lib.pisa_profile_enable.restype = ctypes.c_int
    lib.pisa_profile_report.argtypes = [ctypes.c_char_p, sz, ctypes.POINTER(ctypes.c_float),
                                        ctypes.POINTER(i32), i32, ctypes.POINTER(i32)]
    lib.pisa_profile_report.restype = ctypes.c_int
    lib.pisa_status_string.argtypes = [ctypes.c_int]
    lib.pisa_status_string.restype = ctypes.c_char_p
    lib.pisa_last_error.argtypes = []
    lib.pisa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(func: str, status: int):
    if status != PISA_OK:
        lib = load()
        raise PisaError(func, status, lib.pisa_last_error().decode())
