"""ctypes loader for libcompact_attn.so (the HIP library built in-tree).

There is no fallback: if the library is missing or fails to load, every call
raises.  Build it with ``python -m chunked_prefill_sparse_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcompact_attn.so")

CA_OK = 0
CA_F32 = 0
CA_BF16 = 1
CA_BLOCK = 64
CA_MAX_BATCH = 128
CA_MAX_SPLITS = 16
CA_STATIC_SCRATCH_BYTES = 64 << 20
CA_ERR_TOO_LARGE = 6

EXPORTED = (
    "ca_build_union_tables",
    "ca_build_union_tables_devlen",
    "ca_chunk_attention",
    "ca_chunk_attention_devlen",
    "ca_chunk_attention_stamped",
    "ca_chunk_attention_rows",
    "ca_chunk_attention_split",
    "ca_chunk_attention_split_noalloc",
    "ca_chunk_attention_workspace_size",
    "ca_chunk_attention_balanced",
    "ca_chunk_attention_balanced_workspace_size",
    "ca_tables_to_csr",
    "ca_check_tables",
    "ca_compact_kv",
    "ca_append_kv",
    "ca_pool_blocks",
    "ca_block_mask_topk",
    "ca_select_chunk",
    "ca_append_select_chunk",
    "ca_select_chunk_devlen",
    "ca_append_select_chunk_devlen",
    "ca_status_string",
    "ca_last_hip_error",
)

_lock = threading.Lock()
_lib = None

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_i32p = ctypes.POINTER(ctypes.c_int32)


def _declare(lib):
    lib.ca_build_union_tables.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _i32p, _i32p,
                                          _vp, _vp, _vp]
    lib.ca_build_union_tables.restype = _i32
    lib.ca_build_union_tables_devlen.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                                 _vp, _vp, _vp]
    lib.ca_build_union_tables_devlen.restype = _i32
    lib.ca_chunk_attention.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32p, _i32p, _i32, _i32,
                                       _i32, _i32, _i64, _i32, _i32, ctypes.c_float, _i32, _vp,
                                       _vp, _vp]
    lib.ca_chunk_attention.restype = _i32
    lib.ca_chunk_attention_devlen.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32,
                                              _i32, _i32, _i32, _i64, _i32, _i32, ctypes.c_float,
                                              _i32, _vp, _vp, _vp]
    lib.ca_chunk_attention_devlen.restype = _i32
    lib.ca_chunk_attention_stamped.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32p, _i32p, _i32,
                                               _i32, _i32, _i32, _i64, _i32, _i32,
                                               ctypes.c_float, _i32, _vp, _vp, _vp, _i32,
                                               ctypes.POINTER(ctypes.c_int), _vp]
    lib.ca_chunk_attention_stamped.restype = _i32
    lib.ca_chunk_attention_rows.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32p, _i32p,
                                            _i32, _i32, _i32, _i32, _i64, _i32, _i32,
                                            ctypes.c_float, _i32, _vp, _vp, _vp]
    lib.ca_chunk_attention_rows.restype = _i32
    lib.ca_chunk_attention_split.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32p, _i32p, _i32,
                                             _i32, _i32, _i32, _i64, _i32, _i32, ctypes.c_float,
                                             _i32, _i32, _vp, ctypes.c_size_t, _vp, _vp, _vp]
    lib.ca_chunk_attention_split.restype = _i32
    lib.ca_chunk_attention_split_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32p, _i32p,
                                                     _i32, _i32, _i32, _i32, _i64, _i32, _i32,
                                                     ctypes.c_float, _i32, _i32, _vp, _vp, _vp]
    lib.ca_chunk_attention_split_noalloc.restype = _i32
    lib.ca_chunk_attention_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32]
    lib.ca_chunk_attention_workspace_size.restype = ctypes.c_size_t
    lib.ca_chunk_attention_balanced.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32p, _i32p, _i32,
                                                _i32, _i32, _i32, _i64, _i32, _i32,
                                                ctypes.c_float, _i32, _vp, ctypes.c_size_t, _vp,
                                                _vp, _vp]
    lib.ca_chunk_attention_balanced.restype = _i32
    lib.ca_chunk_attention_balanced_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32]
    lib.ca_chunk_attention_balanced_workspace_size.restype = ctypes.c_size_t
    lib.ca_tables_to_csr.argtypes = [_vp, _vp, _i32, _i32, _i32, _i64, _vp, _vp, _vp]
    lib.ca_tables_to_csr.restype = _i32
    lib.ca_check_tables.argtypes = [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]
    lib.ca_check_tables.restype = _i32
    lib.ca_compact_kv.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32p, _i32p, _i32, _i32, _i64, _i32,
                                  _i32, _vp, _vp, _vp, _vp]
    lib.ca_compact_kv.restype = _i32
    lib.ca_append_kv.argtypes = [_vp, _vp, _i32, _i32, _i32, _i64, _i32, _i32, _i32p, _i32p, _vp,
                                 _vp, _vp]
    lib.ca_append_kv.restype = _i32
    lib.ca_pool_blocks.argtypes = [_vp, _i32, _i32, _i32, _i64, _i32, _i32p, _i32p, _vp, _i32,
                                   _vp]
    lib.ca_pool_blocks.restype = _i32
    lib.ca_block_mask_topk.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32p, _i32p,
                                       _i32, _i32, _vp, _vp, _vp]
    lib.ca_block_mask_topk.restype = _i32
    lib.ca_select_chunk.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32p,
                                    _i32p, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp,
                                    _vp]
    lib.ca_select_chunk.restype = _i32
    lib.ca_append_select_chunk.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                           _i64, _i32, _i32p, _i32p, _i32, _i32, _vp, _i32, _vp,
                                           _i32, _vp, _vp, _vp, _vp, _vp]
    lib.ca_append_select_chunk.restype = _i32
    lib.ca_select_chunk_devlen.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _i32,
                                           _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _vp,
                                           _vp, _vp, _vp]
    lib.ca_select_chunk_devlen.restype = _i32
    lib.ca_append_select_chunk_devlen.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                                  _i32, _i32, _i64, _i32, _vp, _vp, _i32, _i32,
                                                  _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp]
    lib.ca_append_select_chunk_devlen.restype = _i32
    lib.ca_status_string.argtypes = [_i32]
    lib.ca_status_string.restype = ctypes.c_char_p
    lib.ca_last_hip_error.argtypes = []
    lib.ca_last_hip_error.restype = ctypes.c_char_p


def lib():
    """The loaded library (loaded once).  Raises RuntimeError if it is not built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m chunked_prefill_sparse_amd.build` (hipcc, gfx950)")
                handle = ctypes.CDLL(LIB_PATH)
                _declare(handle)
                _lib = handle
    return _lib


class CompactAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        l_ = lib()
        msg = l_.ca_status_string(status).decode()
        if status == 5:
            msg += f" [{l_.ca_last_hip_error().decode()}]"
        super().__init__(f"{where}: {msg}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != CA_OK:
        raise CompactAttnError(status, where)


def int_array(values):
    arr = (ctypes.c_int32 * len(values))(*[int(v) for v in values])
    return arr
