"""CPU oracle for the block-sparse mixed-precision attention path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check in
__graft_entry__ and by bench.py's cpu_baseline leg, never by the product
package.  The arithmetic lives in oracle.cpp (plain C++, double precision,
written from the pages, sharing nothing with the GPU library); this module only
marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

from .build import build, library_path

_lib = None

i32, i64, f32, f64 = C.c_int32, C.c_int64, C.c_float, C.c_double
P = C.c_void_p


def load() -> C.CDLL:
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIBRARY") or library_path()  # (a sanitizer-checked build)
        if not os.path.exists(path):
            build()
        lib = C.CDLL(path)
        sig = {
            "oracle_kv_formula_bytes": (i64, [i64] * 6),
            "oracle_tile_action": (C.c_int, [i64] * 4),
            "oracle_bf16_to_float": (f32, [C.c_uint16]),
            "oracle_float_to_bf16": (C.c_uint16, [f32]),
            "oracle_quantize_rows": (None, [P, i64, C.c_int, C.c_int, P, P]),
            "oracle_pack_nibbles": (None, [P, i64, P]),
            "oracle_dense_attention": (None, [P, P, P, i64, i64, C.c_int, C.c_int, P, f64, P]),
            "oracle_schedule_bytes": (i64, [i64, i64, i64]),
            "oracle_build_schedule": (C.c_int, [C.c_int] * 5 + [i64, P, P, P, i64]),
            "oracle_prefill": (C.c_int, [C.c_int] * 5 + [i64, P, P, P, P, P, f32, C.c_int, P, i64, P, P, C.c_int]),
            "oracle_cache_bytes": (i64, [C.c_int] * 5 + [i64, P, P, C.c_int]),
            "oracle_pack_cache": (C.c_int, [C.c_int] * 5 + [i64, i64, P, P, C.c_int, P, P, P, i64]),
            "oracle_decode": (C.c_int, [C.c_int] * 5 + [i64, i64, P, P, C.c_int, P, P, P, f32, P, C.c_int]),
            "oracle_policy_cost": (f64, [i64, C.c_int, i64, i64, f64, f64]),
            "oracle_paged_table": (i64, [C.c_int] * 5 + [i64, P, P, P, P, C.c_int, i64, P, P, i64, P, P, i64,
                                                        C.POINTER(i64)]),
            "oracle_pack_paged": (C.c_int, [C.c_int] * 5 + [i64, i64, P, P, P, C.c_int, P, P, P, P, i64]),
            "oracle_block_summaries": (C.c_int, [C.c_int] * 5 + [i64, i64, P, P, C.c_int, P, P, P, P, P, C.c_int]),
            "oracle_skip_masks": (C.c_int, [C.c_int] * 5 + [i64, i64, P, P, C.c_int, P, P, P, f32, P, C.c_int]),
            "oracle_decode_skip": (C.c_int, [C.c_int] * 5 + [i64, i64, P, P, C.c_int, P, P, P, P, f32, P,
                                                           C.c_int]),
            "oracle_allocate_policy": (C.c_int, [i64, C.c_int, C.c_int, C.c_int, P, f64, f64, f64, P, P,
                                                 C.POINTER(f64), C.POINTER(f64)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def nthreads() -> int:
    """Worker threads: the cores this process may run on, capped by OMP_NUM_THREADS
    when set (else by 16, a one-GPU share of a multi-GPU host)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "16"))
    except ValueError:
        cap = 16
    return max(1, min(avail, cap))


# ------------------------------------------------------------------ helpers
def kv_formula_bytes(L: int, h: int, d_h: int, n: int, b: int, p: int) -> int:
    return int(load().oracle_kv_formula_bytes(L, h, d_h, n, b, p))


def tile_action(qb: int, kb: int, hi: int, keep: int) -> int:
    """-1 non-causal, 0 skip, 4 int4, 8 int8."""
    return int(load().oracle_tile_action(qb, kb, hi, keep))


def float_to_bf16(x: float) -> int:
    return int(load().oracle_float_to_bf16(x))


def bf16_to_float(b: int) -> float:
    return float(load().oracle_bf16_to_float(b))


def quantize_rows(x_bits: np.ndarray, qmax: int):
    """x bf16 bits [..., d] -> (codes int8 [..., d], scales f32 [...])."""
    x = _c(x_bits, np.uint16)
    d = x.shape[-1]
    rows = x.size // d
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    load().oracle_quantize_rows(_p(x), rows, d, qmax, _p(codes), _p(scales))
    return codes, scales


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    c = _c(codes, np.int8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] // 2,), dtype=np.uint8)
    load().oracle_pack_nibbles(_p(c), c.size, _p(out))
    return out


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, scale: float) -> np.ndarray:
    q, k, v = _c(q, np.float64), _c(k, np.float64), _c(v, np.float64)
    m = _c(mask, np.uint8)
    assert q.shape[1] == k.shape[1] and k.shape[0] == v.shape[0] and m.shape == (q.shape[0], k.shape[0])
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    load().oracle_dense_attention(_p(q), _p(k), _p(v), q.shape[0], k.shape[0], q.shape[1], v.shape[1],
                                  _p(m), scale, _p(out))
    return out


# ------------------------------------------------------------------ schedule
def build_schedule(batch, n_q_heads, n_kv_heads, head_dim, block, seq_len, hi, keep) -> np.ndarray:
    hi, keep = _c(hi, np.int32), _c(keep, np.int32)
    nb = (seq_len + block - 1) // block
    nbytes = int(load().oracle_schedule_bytes(batch, n_q_heads, nb))
    out = np.zeros(nbytes // 4, dtype=np.int32)
    rc = load().oracle_build_schedule(batch, n_q_heads, n_kv_heads, head_dim, block, seq_len,
                                      _p(hi), _p(keep), _p(out), out.size)
    if rc != 0:
        raise RuntimeError("oracle schedule: action map is not of the documented shape")
    return out


# ------------------------------------------------------------------ prefill
def prefill(q, k, v, hi, keep, block: int, sm_scale: float, reference_mode: bool = False,
            units: Optional[Sequence[tuple[int, int, int]]] = None, with_lse: bool = False,
            threads: Optional[int] = None):
    """q [b][Hq][n][d], k, v [b][Hkv][n][d] bf16 bits. Returns out (and lse);
    rows of units not selected are NaN."""
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    b, hq, n, d = q.shape
    hk = k.shape[1]
    hi, keep = _c(hi, np.int32), _c(keep, np.int32)
    out = np.full(q.shape, np.nan, dtype=np.float32)
    lse = np.full(q.shape[:-1], np.nan, dtype=np.float32) if with_lse else None
    u = None if units is None else _c(np.asarray(units).reshape(-1, 3), np.int32)
    load().oracle_prefill(b, hq, hk, d, block, n, _p(q), _p(k), _p(v), _p(hi), _p(keep), sm_scale,
                          int(reference_mode), _p(u), -1 if u is None else u.shape[0], _p(out),
                          _p(lse), threads or nthreads())
    return (out, lse) if with_lse else out


# ------------------------------------------------------------------ cache / decode
def cache_bytes(batch, n_q_heads, n_kv_heads, d, block, ctx_len, hi, keep) -> int:
    hi, keep = _c(hi, np.int32), _c(keep, np.int32)
    return int(load().oracle_cache_bytes(batch, n_q_heads, n_kv_heads, d, block, ctx_len,
                                         _p(hi), _p(keep), hi.size))


def pack_cache(k, v, hi, keep, n_q_heads: int, block: int, ctx_len: int) -> np.ndarray:
    k, v = _c(k, np.uint16), _c(v, np.uint16)
    b, hk, n, d = k.shape
    hi, keep = _c(hi, np.int32), _c(keep, np.int32)
    nbytes = cache_bytes(b, n_q_heads, hk, d, block, ctx_len, hi, keep)
    out = np.zeros(nbytes, dtype=np.uint8)
    rc = load().oracle_pack_cache(b, n_q_heads, hk, d, block, n, ctx_len, _p(hi), _p(keep), hi.size,
                                  _p(k), _p(v), _p(out), nbytes)
    if rc != 0:
        raise RuntimeError("oracle pack_cache failed")
    return out


def decode(k, v, q, hi, keep, block: int, ctx_len: int, sm_scale: float, threads: Optional[int] = None):
    """k, v [b][Hkv][n][d], q [b][Hq][d] bf16 bits -> out f32 [b][Hq][d]."""
    k, v, q = _c(k, np.uint16), _c(v, np.uint16), _c(q, np.uint16)
    b, hk, n, d = k.shape
    hq = q.shape[1]
    hi, keep = _c(hi, np.int32), _c(keep, np.int32)
    out = np.empty((b, hq, d), dtype=np.float32)
    load().oracle_decode(b, hq, hk, d, block, n, ctx_len, _p(hi), _p(keep), hi.size, _p(k), _p(v),
                         _p(q), sm_scale, _p(out), threads or nthreads())
    return out


def block_summaries(k, hi, keep, n_q_heads: int, block: int, ctx_len: int, threads: Optional[int] = None):
    """Statistics of every stored record of the cache for ctx_len (record order, rmax =
    cur_block + 1 slots per pair): (lo, hi) int8 [P][rmax][d], smax f32 [P][rmax],
    nmax f64 [P][rmax]."""
    k = _c(k, np.uint16)
    b, hk, n, d = k.shape
    hi, keep = _c(hi, np.int32), _c(keep, np.int32)
    rmax = (ctx_len - 1) // block + 1
    lo = np.zeros((b * hk, rmax, d), np.int8)
    up = np.zeros((b * hk, rmax, d), np.int8)
    smax = np.zeros((b * hk, rmax), np.float32)
    nmax = np.zeros((b * hk, rmax), np.float64)
    load().oracle_block_summaries(b, n_q_heads, hk, d, block, n, ctx_len, _p(hi), _p(keep), hi.size, _p(k), _p(lo),
                                  _p(up), _p(smax), _p(nmax), threads or nthreads())
    return lo, up, smax, nmax


def skip_masks(k, q, hi, keep, block: int, ctx_len: int, thresholds, sm_scale: float,
               threads: Optional[int] = None) -> np.ndarray:
    """Per stored record (record order), bit i = query head g*G + i keeps it: uint32 [P][rmax]."""
    k, q = _c(k, np.uint16), _c(q, np.uint16)
    b, hk, n, d = k.shape
    hq = q.shape[1]
    hi, keep = _c(hi, np.int32), _c(keep, np.int32)
    th = _c(thresholds, np.float32)
    assert th.size == b * hq
    rmax = (ctx_len - 1) // block + 1
    masks = np.zeros((b * hk, rmax), np.uint32)
    if load().oracle_skip_masks(b, hq, hk, d, block, n, ctx_len, _p(hi), _p(keep), hi.size, _p(k), _p(q), _p(th),
                                sm_scale, _p(masks), threads or nthreads()):
        raise ValueError("more than 32 query heads per KV head")
    return masks


def decode_skip(k, v, q, hi, keep, block: int, ctx_len: int, thresholds, sm_scale: float,
                threads: Optional[int] = None):
    """Decode with dynamic block skipping: out f32 [b][Hq][d]."""
    k, v, q = _c(k, np.uint16), _c(v, np.uint16), _c(q, np.uint16)
    b, hk, n, d = k.shape
    hq = q.shape[1]
    hi, keep = _c(hi, np.int32), _c(keep, np.int32)
    th = _c(thresholds, np.float32)
    assert th.size == b * hq
    out = np.empty((b, hq, d), dtype=np.float32)
    if load().oracle_decode_skip(b, hq, hk, d, block, n, ctx_len, _p(hi), _p(keep), hi.size, _p(k), _p(v), _p(q),
                                 _p(th), sm_scale, _p(out), threads or nthreads()):
        raise ValueError("more than 32 query heads per KV head")
    return out


def paged_table(batch: int, n_q_heads: int, n_kv_heads: int, d: int, block: int, ctx_len, hi, keep,
                n_pages: int, old_table: Optional[np.ndarray], free_pages, released_cap: int = 1 << 20,
                seq_ids=None):
    """Page table bytes (uint8), pages taken, pages released.  ctx_len: one length, or
    a sequence of lengths per batch element (variable-length table, where seq_ids
    optionally names each slot's sequence)."""
    hi, keep = _c(hi, np.int32), _c(keep, np.int32)
    fp = _c(free_pages, np.int32)
    P_ = batch * n_kv_heads
    lens = None if np.isscalar(ctx_len) else _c(ctx_len, np.int64)
    rmax = ((int(ctx_len) if lens is None else int(lens.max())) - 1) // block + 1
    table = np.zeros(64 + 64 * P_ + 4 * P_ * rmax, np.uint8)
    rel = np.zeros(max(released_cap, 1), np.int32)
    nrel = C.c_int64(0)
    ot = None if old_table is None else _c(old_table, np.uint8)
    sids = None if seq_ids is None else _c(seq_ids, np.int64)
    taken = load().oracle_paged_table(batch, n_q_heads, n_kv_heads, d, block, 0 if lens is not None else ctx_len,
                                      _p(lens), _p(sids), _p(hi), _p(keep), hi.size, n_pages, _p(ot), _p(fp), fp.size,
                                      _p(table), _p(rel), released_cap, C.byref(nrel))
    if taken < 0:
        raise ValueError("too few free pages" if taken == -1 else "released list too small")
    return table, int(taken), rel[:nrel.value].copy()


def pack_paged(k, v, hi, keep, n_q_heads: int, block: int, ctx_len, table: np.ndarray, pool: np.ndarray):
    """Writes every stored record of the cache for ctx_len (one length, or one per batch
    element) into its page of pool (uint8)."""
    k, v = _c(k, np.uint16), _c(v, np.uint16)
    b, hk, n, d = k.shape
    hi, keep = _c(hi, np.int32), _c(keep, np.int32)
    t = _c(table, np.uint8)
    lens = None if np.isscalar(ctx_len) else _c(ctx_len, np.int64)
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    if load().oracle_pack_paged(b, n_q_heads, hk, d, block, n, 0 if lens is not None else ctx_len, _p(lens), _p(hi),
                                _p(keep), hi.size, _p(k), _p(v), _p(t), _p(pool), pool.size):
        raise ValueError("table and pool do not match")
    return pool


def policy_cost(n: int, block: int, hi: int, keep: int, c8: float = 1.0, c4: float = 1.0) -> float:
    """Cost of one head's (hi, keep): its kept tiles as whole blocks at each precision's pair cost."""
    return float(load().oracle_policy_cost(n, block, hi, keep, c8, c4))


def allocate_policy(n: int, block: int, err: np.ndarray, budget: float, c8: float = 1.0, c4: float = 1.0):
    """Greedy per-head (hi, keep) under a cost budget; returns (hi, keep, total_cost, total_err),
    or raises ValueError when the budget is below the protected-only cost."""
    err = _c(err, np.float64)
    H, K = err.shape[0], err.shape[1] - 1
    hi = np.zeros(H, np.int32)
    keep = np.zeros(H, np.int32)
    tc, te = C.c_double(0.0), C.c_double(0.0)
    if load().oracle_allocate_policy(n, block, H, K, _p(err), c8, c4, budget, _p(hi), _p(keep), C.byref(tc),
                                     C.byref(te)):
        raise ValueError("budget below the protected-only cost")
    return hi, keep, tc.value, te.value

