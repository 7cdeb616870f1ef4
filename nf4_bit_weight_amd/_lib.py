"""ctypes loader for libnf4.so (the C ABI declared in include/nf4.h).

The library must be built in-tree first (`python -m nf4_bit_weight_amd.build`
or __graft_entry__.build()).  There is no fallback: if the shared library is
missing or does not load, every entry point raises.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnf4.so")

# status codes (nf4.h)
NF4_OK = 0
NF4_ERR_NULL = -1
NF4_ERR_SHAPE = -2
NF4_ERR_UNSUPPORTED = -3
NF4_ERR_ALIGN = -4
NF4_ERR_WORKSPACE = -5
NF4_ERR_HIP = -6
NF4_ERR_DTYPE = -7
NF4_ERR_SCRATCH = -8

NF4_NOALLOC_SCRATCH_BYTES = 64 << 20

NF4_DTYPE_F32 = 0
NF4_DTYPE_BF16 = 1

NF4_OP_QUANTIZE = 0
NF4_OP_MATMUL_FWD = 1
NF4_OP_MATMUL_BWD_INPUT = 2
NF4_OP_GROUPED_FWD = 3
NF4_OP_GROUPED_BWD_INPUT = 4
NF4_OP_MATMUL_FWD_8BIT = 5
NF4_OP_MATMUL_BWD_INPUT_8BIT = 6

PATHS = ("quantize", "dequantize", "fwd_tiled", "fwd_small_m", "bwd_tiled",
         "splitk_reduce", "grouped_fwd", "grouped_bwd", "fwd_8bit", "bwd_8bit")

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_int = ctypes.c_int
_size = ctypes.c_size_t

_W = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64]   # packed .. nested_code256, N, K

# name -> (restype, argtypes); the full exported surface of nf4.h
SIGNATURES = {
    "nf4_quantize": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _size, _vp]),
    "nf4_dequantize": (_int, [*_W, _int, _vp, _vp]),
    "nf4_matmul_fwd": (_int, [_vp, _i64, *_W, _vp, _vp, _size, _vp]),
    "nf4_matmul_bwd_input": (_int, [_vp, _i64, *_W, _vp, _vp, _size, _vp]),
    "nf4_matmul_fwd_noalloc": (_int, [_vp, _i64, *_W, _vp, _vp]),
    "nf4_quantize_8bit": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _size, _vp]),
    "nf4_dequantize_8bit": (_int, [*_W, _int, _vp, _vp]),
    "nf4_matmul_fwd_8bit": (_int, [_vp, _i64, *_W, _vp, _vp, _size, _vp]),
    "nf4_matmul_bwd_input_8bit": (_int, [_vp, _i64, *_W, _vp, _vp, _size, _vp]),
    "nf4_grouped_matmul_fwd_8bit": (_int, [_vp, _vp, _i32, _i64, *_W, _vp, _vp, _size, _vp]),
    "nf4_grouped_matmul_bwd_input_8bit": (_int, [_vp, _vp, _i32, _i64, *_W, _vp, _vp, _size, _vp]),
    "nf4_grouped_matmul_fwd": (_int, [_vp, _vp, _i32, _i64, *_W, _vp, _vp, _size, _vp]),
    "nf4_grouped_matmul_bwd_input": (_int, [_vp, _vp, _i32, _i64, *_W, _vp, _vp, _size, _vp]),
    "nf4_workspace_bytes": (_size, [_int, _i64, _i64, _i64, _i32]),
    "nf4_packed_bytes": (_i64, [_i64, _i64]),
    "nf4_absmax_count": (_i64, [_i64, _i64]),
    "nf4_nested_count": (_i64, [_i64, _i64]),
    "nf4_path_count": (_i64, [_int]),
    "nf4_reset_path_counts": (None, []),
    "nf4_status_str": (ctypes.c_char_p, [_int]),
    "nf4_version": (ctypes.c_char_p, []),
}

_lib = None


class NF4Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libnf4.so once; raise if it is missing (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m nf4_bit_weight_amd.build`")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    _lib = handle
    return handle


def status_str(status: int) -> str:
    return lib().nf4_status_str(status).decode()


def check(fn: str, status: int) -> None:
    if status != NF4_OK:
        raise NF4Error(fn, status, status_str(status))
