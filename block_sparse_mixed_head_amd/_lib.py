"""ctypes binding of libtria.so (argument marshalling only).

The names mirror the C ABI in include/tria.h.  Every compute step runs in the HIP
kernels behind it; if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# TRIA_LIBRARY: another build of the same library (the sanitizer-checked host build)
LIB_PATH = os.environ.get("TRIA_LIBRARY") or os.path.join(HERE, "libtria.so")

TRIA_OK, TRIA_ERR_INVALID_ARG, TRIA_ERR_UNSUPPORTED, TRIA_ERR_BUFFER_TOO_SMALL, TRIA_ERR_HIP = range(5)
SCHED_HEADER_BYTES = 64
SCHED_UNIT_BYTES = 32


class TriaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"tria status {status}: {msg}")
        self.status = status


class Dims(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("block", C.c_int32), ("reserved", C.c_int32),
                ("seq_len", C.c_int64)]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(block_sparse_mixed_head_amd/build.py) first")
    lib = C.CDLL(LIB_PATH)
    P, sz, i32, i64, f32 = C.c_void_p, C.c_size_t, C.c_int32, C.c_int64, C.c_float
    D = C.POINTER(Dims)
    sigs = {
        "tria_last_error": (C.c_char_p, []),
        "tria_version": (i32, []),
        "tria_build_policy": (C.c_int, [D, P, P, i32, P, sz, C.POINTER(sz)]),
        "tria_quantize_qk": (C.c_int, [D, P, P] + [P] * 8 + [P]),
        "tria_prefill": (C.c_int, [D, P, sz] + [P] * 8 + [P, f32, P, P, P]),
        "tria_prefill_bf16q": (C.c_int, [D, P, sz, P] + [P] * 4 + [P, f32, P, P, P]),
        "tria_quantize_k": (C.c_int, [D, P] + [P] * 4 + [P]),
        "tria_build_policy_varlen": (C.c_int, [D, P, P, i32, i32, P, P, sz, C.POINTER(sz)]),
        "tria_prefill_varlen": (C.c_int, [D, i32, P, P, sz] + [P] * 8 + [P, f32, P, P, P]),
        "tria_kv_cache_bytes": (C.c_int, [D, P, P, i32, i64, C.POINTER(sz)]),
        "tria_pack_kv_cache": (C.c_int, [D, P, P, i32, i64, P, P, P, sz, P]),
        "tria_update_kv_cache": (C.c_int, [D, P, P, i32, i64, P, P, P, sz, P, sz, P]),
        "tria_kv_cache_bytes_varlen": (C.c_int, [D, P, P, i32, P, C.POINTER(sz)]),
        "tria_pack_kv_cache_varlen": (C.c_int, [D, P, P, i32, P, P, P, P, sz, P]),
        "tria_decode_varlen": (C.c_int, [D, P, sz, P, f32, P, P, sz, P]),
        "tria_check_cache": (C.c_int, [D, P, sz, i64]),
        "tria_decode_workspace_bytes": (C.c_int, [D, i64, C.POINTER(sz)]),
        "tria_decode": (C.c_int, [D, P, sz, i64, P, f32, P, P, sz, P]),
        "tria_decode_noalloc": (C.c_int, [D, P, sz, i64, P, f32, P, P]),
        "tria_policy_cost": (C.c_int, [D, i32, i32, C.c_double, C.c_double, C.POINTER(C.c_double)]),
        "tria_allocate_policy": (C.c_int, [D, i32, i32, P, C.c_double, C.c_double, C.c_double, P, P,
                                           C.POINTER(C.c_double), C.POINTER(C.c_double)]),
        "tria_block_summaries_bytes": (C.c_int, [D, i64, C.POINTER(sz)]),
        "tria_build_block_summaries": (C.c_int, [D, P, sz, i64, P, sz, P]),
        "tria_skip_masks": (C.c_int, [D, P, sz, i64, P, sz, P, P, f32, P, sz, P]),
        "tria_decode_skip_workspace_bytes": (C.c_int, [D, i64, C.POINTER(sz)]),
        "tria_decode_skip": (C.c_int, [D, P, sz, i64, P, sz, P, P, f32, P, P, sz, P]),
        "tria_paged_page_bytes": (C.c_int, [D, C.POINTER(sz)]),
        "tria_paged_table_bytes": (C.c_int, [D, i64, C.POINTER(sz)]),
        "tria_build_paged_table": (C.c_int, [D, P, P, i32, i64, i64, P, sz, P, i32, P, sz, C.POINTER(i32), P, i32,
                                             C.POINTER(i32)]),
        "tria_build_paged_table_varlen": (C.c_int, [D, P, P, i32, P, P, i64, P, sz, P, i32, P, sz, C.POINTER(i32), P,
                                                    i32, C.POINTER(i32)]),
        "tria_pack_kv_cache_paged": (C.c_int, [D, P, P, i32, i64, P, P, P, sz, P, sz, P, sz, P]),
        "tria_decode_paged": (C.c_int, [D, P, sz, P, sz, i64, P, f32, P, P, sz, P]),
        "tria_pack_kv_cache_paged_varlen": (C.c_int, [D, P, P, i32, P, P, P, P, sz, P, sz, P, sz, P]),
        "tria_build_block_summaries_paged": (C.c_int, [D, P, sz, P, sz, i64, P, sz, P]),
        "tria_build_block_summaries_varlen": (C.c_int, [D, P, sz, P, sz, P]),
        "tria_build_block_summaries_paged_varlen": (C.c_int, [D, P, sz, P, sz, P, sz, P]),
        "tria_decode_skip_paged_varlen": (C.c_int, [D, P, sz, P, sz, P, sz, P, P, f32, P, P, sz, P]),
        "tria_decode_skip_varlen": (C.c_int, [D, P, sz, P, sz, P, P, f32, P, P, sz, P]),
        "tria_decode_skip_paged": (C.c_int, [D, P, sz, P, sz, i64, P, sz, P, P, f32, P, P, sz, P]),
        "tria_decode_paged_varlen": (C.c_int, [D, P, sz, P, sz, P, f32, P, P, sz, P]),
        "tria_peak_mfma": (C.c_int, [i32, i32, P, C.POINTER(C.c_double), P]),
        "tria_peak_read": (C.c_int, [P, i64, P, C.POINTER(C.c_double), P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()

EXPORTED = ["tria_last_error", "tria_version", "tria_build_policy", "tria_quantize_qk", "tria_prefill",
            "tria_prefill_bf16q", "tria_quantize_k",
            "tria_build_policy_varlen", "tria_prefill_varlen",
            "tria_kv_cache_bytes", "tria_pack_kv_cache", "tria_update_kv_cache", "tria_check_cache",
            "tria_kv_cache_bytes_varlen", "tria_pack_kv_cache_varlen", "tria_decode_varlen",
            "tria_decode_workspace_bytes", "tria_decode", "tria_decode_noalloc", "tria_policy_cost",
            "tria_allocate_policy",
            "tria_block_summaries_bytes", "tria_build_block_summaries", "tria_skip_masks",
            "tria_decode_skip_workspace_bytes", "tria_decode_skip", "tria_paged_page_bytes", "tria_paged_table_bytes",
            "tria_build_paged_table", "tria_build_paged_table_varlen", "tria_pack_kv_cache_paged", "tria_decode_paged",
            "tria_pack_kv_cache_paged_varlen", "tria_decode_paged_varlen", "tria_build_block_summaries_paged",
            "tria_decode_skip_paged", "tria_build_block_summaries_varlen", "tria_decode_skip_varlen",
            "tria_build_block_summaries_paged_varlen", "tria_decode_skip_paged_varlen", "tria_peak_mfma",
            "tria_peak_read"]
PEAK_READ_ALIGN = 8192 * 8 * 1024
PEAK_SINK_INTS = 8192


def check(status: int) -> None:
    if status != TRIA_OK:
        raise TriaError(status, lib.tria_last_error().decode())


def dims(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, block: int, seq_len: int) -> Dims:
    return Dims(batch, n_q_heads, n_kv_heads, head_dim, block, 0, seq_len)
