"""ctypes mirror of include/mla_decode.h.

Loads the in-tree libmla_decode.so and fails loudly when it is missing: there
is no fallback implementation behind this binding.
"""

from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
# (MLA_DECODE_LIBRARY names another build of the same library, such as the
# sanitized host build the CPU tests load)
LIB_PATH = os.environ.get("MLA_DECODE_LIBRARY") or os.path.join(HERE, "libmla_decode.so")

MLA_OK = 0
MLA_ERR_NULL_POINTER = 1
MLA_ERR_BAD_SHAPE = 2
MLA_ERR_BAD_STRIDE = 3
MLA_ERR_UNSUPPORTED = 4
MLA_ERR_WORKSPACE_TOO_SMALL = 5
MLA_ERR_HIP = 6
MLA_ERR_BAD_ARGUMENT = 7
MLA_ERR_SCRATCH_TOO_SMALL = 8
NOALLOC_SCRATCH_BYTES = 64 << 20
TILE_MD_INTS = 8
KV_BF16 = 0
KV_FP8_E4M3 = 1
ROWS_PER_WORKGROUP = 128
MAX_ROWS = 1024

EXPORTS = (
    "mla_status_string",
    "mla_decode_params_size",
    "mla_default_num_parts",
    "mla_get_metadata",
    "mla_plan_host",
    "mla_workspace_size",
    "mla_decode_with_kvcache",
    "mla_decode_with_kvcache_noalloc",
    "mla_append_kv",
    "mla_copy_blocks",
)

c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_p = ctypes.c_void_p
c_i32p = ctypes.POINTER(ctypes.c_int32)


class DecodeParams(ctypes.Structure):
    _fields_ = [
        ("q", c_p), ("q_batch_stride", c_i64), ("q_seq_stride", c_i64), ("q_head_stride", c_i64),
        ("batch", c_i32), ("s_q", c_i32), ("h_q", c_i32),
        ("k_cache", c_p), ("k_block_stride", c_i64), ("k_row_stride", c_i64), ("k_head_stride", c_i64),
        ("num_blocks", c_i32), ("block_size", c_i32), ("h_kv", c_i32), ("d", c_i32),
        ("block_table", c_p), ("block_table_stride", c_i64), ("max_blocks_per_seq", c_i32),
        ("cache_seqlens", c_p),
        ("dv", c_i32), ("softmax_scale", ctypes.c_float), ("causal", c_i32),
        ("tile_md", c_p), ("num_splits", c_p), ("num_parts", c_i32),
        ("workspace", c_p), ("workspace_bytes", ctypes.c_size_t),
        ("out", c_p), ("out_batch_stride", c_i64), ("out_seq_stride", c_i64), ("out_head_stride", c_i64),
        ("lse", c_p), ("lse_batch_stride", c_i64), ("lse_seq_stride", c_i64), ("lse_head_stride", c_i64),
        ("kv_dtype", c_i32), ("kv_scale", ctypes.c_float),
    ]


class MLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lock = threading.Lock()
_lib = None


def load():
    """The loaded library (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m paged_mla_decode_04_amd.build, or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        lib.mla_status_string.restype = ctypes.c_char_p
        lib.mla_status_string.argtypes = [ctypes.c_int]
        lib.mla_decode_params_size.restype = ctypes.c_size_t
        lib.mla_decode_params_size.argtypes = []
        lib.mla_default_num_parts.restype = ctypes.c_int
        lib.mla_default_num_parts.argtypes = [ctypes.c_int, c_i32, c_i32, c_i32p]
        lib.mla_get_metadata.restype = ctypes.c_int
        lib.mla_get_metadata.argtypes = [c_p, c_i32, c_i32, c_i32, c_i32, c_p, c_p, c_p]
        lib.mla_plan_host.restype = ctypes.c_int
        lib.mla_plan_host.argtypes = [c_p, c_i32, c_i32, c_i32, c_i32, c_p, c_p]
        lib.mla_workspace_size.restype = ctypes.c_int
        lib.mla_workspace_size.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                           ctypes.POINTER(ctypes.c_size_t)]
        lib.mla_decode_with_kvcache.restype = ctypes.c_int
        lib.mla_decode_with_kvcache.argtypes = [ctypes.POINTER(DecodeParams), c_p]
        lib.mla_decode_with_kvcache_noalloc.restype = ctypes.c_int
        lib.mla_decode_with_kvcache_noalloc.argtypes = [ctypes.POINTER(DecodeParams), c_p]
        lib.mla_append_kv.restype = ctypes.c_int
        lib.mla_append_kv.argtypes = [c_p, c_i64, c_p, c_i64, c_p, c_i32, c_p, c_i32, c_i64, c_i64, c_p]
        lib.mla_copy_blocks.restype = ctypes.c_int
        lib.mla_copy_blocks.argtypes = [c_p, c_i32, c_i64, c_i64, c_p, c_i32, c_i64, c_i64, c_p, c_i32, c_p]
        if lib.mla_decode_params_size() != ctypes.sizeof(DecodeParams):
            raise RuntimeError("mla_decode_params layout mismatch between the binding and the library")
        _lib = lib
        return lib


def status_string(status: int) -> str:
    try:
        return load().mla_status_string(int(status)).decode()
    except Exception:  # library missing: still produce a message
        return "unknown"


def check(status: int, what: str) -> None:
    if status != MLA_OK:
        if status in (MLA_ERR_BAD_SHAPE, MLA_ERR_BAD_STRIDE, MLA_ERR_UNSUPPORTED,
                      MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_NULL_POINTER, MLA_ERR_BAD_ARGUMENT,
                      MLA_ERR_SCRATCH_TOO_SMALL):
            raise ValueError(f"{what}: {status_string(status)} (status {status})")
        raise MLAError(status, what)
