"""Block-sparse, mixed-precision (int8 / int4 / skip) causal attention on MI355X.

Thin torch-facing wrappers over the C ABI (include/tria.h, libtria.so).  PyTorch
provides device memory and the current stream; every step of the attention path
runs in the library's HIP kernels.  The five calls of the path:

  build_policy   per-head (hi, keep) -> schedule of per-(b, h, q-block) units
  quantize_qk    per-row int8 / int4 codes and fp32 scales of Q and K
  prefill        fused block-sparse causal attention over the schedule
  pack_kv_cache  compressed int8 / int4 KV cache for one query position
  decode         one-token attention over the compressed cache
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib
from ._lib import TriaError, check, dims as make_dims  # noqa: F401

__all__ = ["Dims", "build_policy", "build_policy_varlen", "quantize_qk", "quantize_k", "prefill", "prefill_bf16q", "prefill_varlen", "kv_cache_bytes", "pack_kv_cache", "update_kv_cache",
           "kv_cache_bytes_varlen", "pack_kv_cache_varlen", "decode_varlen",
           "check_cache", "decode_workspace_bytes", "decode", "block_summaries_bytes", "build_block_summaries",
           "skip_masks", "decode_skip_workspace_bytes", "decode_skip", "paged_page_bytes", "paged_table_bytes",
           "build_paged_table", "pack_kv_cache_paged", "decode_paged", "decode_paged_varlen", "build_block_summaries_paged",
           "decode_skip_paged", "build_block_summaries_varlen", "decode_skip_varlen",
           "build_block_summaries_paged_varlen", "decode_skip_paged_varlen", "policy_cost", "allocate_policy", "peak_mfma", "peak_read", "TriaError",
           "Quantized"]

Dims = _lib.Dims


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _require(t: torch.Tensor, dtype, shape, name: str) -> None:
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous CUDA {dtype} {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()} cuda={t.is_cuda}")


# ------------------------------------------------------------------ (1) policy
def build_policy(d: Dims, hi, keep) -> np.ndarray:
    """Host schedule blob (int32 words) for per-query-head (hi, keep)."""
    hi, keep = _i32(hi), _i32(keep)
    need = C.c_size_t(0)
    check(_lib.lib.tria_build_policy(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi), None, 0,
                                     C.byref(need)))
    out = np.zeros(need.value // 4, dtype=np.int32)
    check(_lib.lib.tria_build_policy(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi),
                                     out.ctypes.data, need.value, C.byref(need)))
    return out


# ------------------------------------------------------------------ (2) quantiser
@dataclass
class Quantized:
    q8: torch.Tensor
    q4: torch.Tensor
    q8s: torch.Tensor
    q4s: torch.Tensor
    k8: torch.Tensor
    k4: torch.Tensor
    k8s: torch.Tensor
    k4s: torch.Tensor


def quantize_qk(d: Dims, q: torch.Tensor, k: torch.Tensor, out: Optional[Quantized] = None) -> Quantized:
    b, hq, hk, hd, n = d.batch, d.n_q_heads, d.n_kv_heads, d.head_dim, d.seq_len
    _require(q, torch.bfloat16, (b, hq, n, hd), "q")
    _require(k, torch.bfloat16, (b, hk, n, hd), "k")
    dev = q.device
    if out is None:
        out = Quantized(
            torch.empty((b, hq, n, hd), dtype=torch.int8, device=dev),
            torch.empty((b, hq, n, hd // 2), dtype=torch.uint8, device=dev),
            torch.empty((b, hq, n), dtype=torch.float32, device=dev),
            torch.empty((b, hq, n), dtype=torch.float32, device=dev),
            torch.empty((b, hk, n, hd), dtype=torch.int8, device=dev),
            torch.empty((b, hk, n, hd // 2), dtype=torch.uint8, device=dev),
            torch.empty((b, hk, n), dtype=torch.float32, device=dev),
            torch.empty((b, hk, n), dtype=torch.float32, device=dev))
    check(_lib.lib.tria_quantize_qk(C.byref(d), _ptr(q), _ptr(k), _ptr(out.q8), _ptr(out.q4), _ptr(out.q8s),
                                    _ptr(out.q4s), _ptr(out.k8), _ptr(out.k4), _ptr(out.k8s), _ptr(out.k4s),
                                    _stream(dev)))
    return out


@dataclass
class QuantizedK:
    k8: torch.Tensor
    k4: torch.Tensor
    k8s: torch.Tensor
    k4s: torch.Tensor


def quantize_k(d: Dims, k: torch.Tensor, out: Optional[QuantizedK] = None) -> QuantizedK:
    """K codes and scales alone (as quantize_qk writes them), for prefill_bf16q."""
    b, hk, hd, n = d.batch, d.n_kv_heads, d.head_dim, d.seq_len
    _require(k, torch.bfloat16, (b, hk, n, hd), "k")
    dev = k.device
    if out is None:
        out = QuantizedK(torch.empty((b, hk, n, hd), dtype=torch.int8, device=dev),
                         torch.empty((b, hk, n, hd // 2), dtype=torch.uint8, device=dev),
                         torch.empty((b, hk, n), dtype=torch.float32, device=dev),
                         torch.empty((b, hk, n), dtype=torch.float32, device=dev))
    check(_lib.lib.tria_quantize_k(C.byref(d), _ptr(k), _ptr(out.k8), _ptr(out.k4), _ptr(out.k8s), _ptr(out.k4s),
                                   _stream(dev)))
    return out


# ------------------------------------------------------------------ (3) prefill
def prefill(d: Dims, sched_dev: torch.Tensor, qz: Quantized, v: torch.Tensor, sm_scale: float,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sched_dev: the build_policy blob copied to the device (any dtype, contiguous)."""
    b, hq, hk, hd, n = d.batch, d.n_q_heads, d.n_kv_heads, d.head_dim, d.seq_len
    _require(v, torch.bfloat16, (b, hk, n, hd), "v")
    if out is None:
        out = torch.empty((b, hq, n, hd), dtype=torch.float32, device=v.device)
    _require(out, torch.float32, (b, hq, n, hd), "out")
    if lse is not None:
        _require(lse, torch.float32, (b, hq, n), "lse")
    nbytes = sched_dev.numel() * sched_dev.element_size()
    check(_lib.lib.tria_prefill(C.byref(d), _ptr(sched_dev), nbytes, _ptr(qz.q8), _ptr(qz.q4), _ptr(qz.q8s),
                                _ptr(qz.q4s), _ptr(qz.k8), _ptr(qz.k4), _ptr(qz.k8s), _ptr(qz.k4s), _ptr(v),
                                float(sm_scale), _ptr(out), _ptr(lse), _stream(v.device)))
    return out


def prefill_bf16q(d: Dims, sched_dev: torch.Tensor, q: torch.Tensor, kz, v: torch.Tensor, sm_scale: float,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None) -> torch.Tensor:
    """prefill with Q as bf16, quantised inside the kernel; kz: QuantizedK (or
    Quantized) holding the K codes and scales."""
    b, hq, hk, hd, n = d.batch, d.n_q_heads, d.n_kv_heads, d.head_dim, d.seq_len
    _require(q, torch.bfloat16, (b, hq, n, hd), "q")
    _require(v, torch.bfloat16, (b, hk, n, hd), "v")
    if out is None:
        out = torch.empty((b, hq, n, hd), dtype=torch.float32, device=v.device)
    _require(out, torch.float32, (b, hq, n, hd), "out")
    if lse is not None:
        _require(lse, torch.float32, (b, hq, n), "lse")
    nbytes = sched_dev.numel() * sched_dev.element_size()
    check(_lib.lib.tria_prefill_bf16q(C.byref(d), _ptr(sched_dev), nbytes, _ptr(q), _ptr(kz.k8), _ptr(kz.k4),
                                      _ptr(kz.k8s), _ptr(kz.k4s), _ptr(v), float(sm_scale), _ptr(out), _ptr(lse),
                                      _stream(v.device)))
    return out


def _cu(cu_seqlens) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))


def build_policy_varlen(d: Dims, hi, keep, cu_seqlens) -> np.ndarray:
    """Schedule blob (int32 words) for sequences packed along the rows of one batch
    element: d.batch == 1, d.seq_len = cu_seqlens[-1]."""
    hi, keep, cu = _i32(hi), _i32(keep), _cu(cu_seqlens)
    need = C.c_size_t(0)
    check(_lib.lib.tria_build_policy_varlen(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi), len(cu) - 1,
                                            cu.ctypes.data, None, 0, C.byref(need)))
    out = np.zeros(need.value // 4, dtype=np.int32)
    check(_lib.lib.tria_build_policy_varlen(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi), len(cu) - 1,
                                            cu.ctypes.data, out.ctypes.data, need.value, C.byref(need)))
    return out


def prefill_varlen(d: Dims, cu_seqlens, sched_dev: torch.Tensor, qz: Quantized, v: torch.Tensor, sm_scale: float,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Prefill of a variable-length batch over a build_policy_varlen blob on the device."""
    hq, hk, hd, n = d.n_q_heads, d.n_kv_heads, d.head_dim, d.seq_len
    cu = _cu(cu_seqlens)
    _require(v, torch.bfloat16, (1, hk, n, hd), "v")
    if out is None:
        out = torch.empty((1, hq, n, hd), dtype=torch.float32, device=v.device)
    _require(out, torch.float32, (1, hq, n, hd), "out")
    if lse is not None:
        _require(lse, torch.float32, (1, hq, n), "lse")
    nbytes = sched_dev.numel() * sched_dev.element_size()
    check(_lib.lib.tria_prefill_varlen(C.byref(d), len(cu) - 1, cu.ctypes.data, _ptr(sched_dev), nbytes,
                                       _ptr(qz.q8), _ptr(qz.q4), _ptr(qz.q8s), _ptr(qz.q4s), _ptr(qz.k8),
                                       _ptr(qz.k4), _ptr(qz.k8s), _ptr(qz.k4s), _ptr(v), float(sm_scale),
                                       _ptr(out), _ptr(lse), _stream(v.device)))
    return out


# ------------------------------------------------------------------ (4) cache
def kv_cache_bytes(d: Dims, hi, keep, ctx_len: int) -> int:
    hi, keep = _i32(hi), _i32(keep)
    out = C.c_size_t(0)
    check(_lib.lib.tria_kv_cache_bytes(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi), ctx_len,
                                       C.byref(out)))
    return out.value


def pack_kv_cache(d: Dims, hi, keep, ctx_len: int, k: torch.Tensor, v: torch.Tensor,
                  cache: Optional[torch.Tensor] = None) -> torch.Tensor:
    b, hk, hd, n = d.batch, d.n_kv_heads, d.head_dim, d.seq_len
    _require(k, torch.bfloat16, (b, hk, n, hd), "k")
    _require(v, torch.bfloat16, (b, hk, n, hd), "v")
    hi, keep = _i32(hi), _i32(keep)
    nbytes = kv_cache_bytes(d, hi, keep, ctx_len)
    if cache is None:
        cache = torch.empty(nbytes, dtype=torch.uint8, device=k.device)
    check(_lib.lib.tria_pack_kv_cache(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi), ctx_len, _ptr(k),
                                      _ptr(v), _ptr(cache), cache.numel(), _stream(k.device)))
    return cache


def update_kv_cache(d: Dims, hi, keep, ctx_len: int, k: torch.Tensor, v: torch.Tensor, cache: torch.Tensor,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The cache for ctx_len from `cache`, the one packed for ctx_len - 1 from the same
    k, v and policy.  Within a block it is updated in place (returned as is); when
    token ctx_len - 1 starts a new block the records move and the result goes to
    `out` (allocated when None)."""
    b, hk, hd, n = d.batch, d.n_kv_heads, d.head_dim, d.seq_len
    _require(k, torch.bfloat16, (b, hk, n, hd), "k")
    _require(v, torch.bfloat16, (b, hk, n, hd), "v")
    _require(cache, torch.uint8, (cache.numel(),), "cache")
    hi, keep = _i32(hi), _i32(keep)
    if (ctx_len - 1) % d.block != 0:
        dst = cache
    else:
        dst = out if out is not None else torch.empty(kv_cache_bytes(d, hi, keep, ctx_len), dtype=torch.uint8,
                                                      device=k.device)
    check(_lib.lib.tria_update_kv_cache(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi), ctx_len, _ptr(k),
                                        _ptr(v), _ptr(cache), cache.numel(), _ptr(dst), dst.numel(),
                                        _stream(k.device)))
    return dst


def kv_cache_bytes_varlen(d: Dims, hi, keep, ctx_lens) -> int:
    hi, keep, cl = _i32(hi), _i32(keep), _cu(ctx_lens)
    out = C.c_size_t(0)
    check(_lib.lib.tria_kv_cache_bytes_varlen(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi), cl.ctypes.data,
                                              C.byref(out)))
    return out.value


def pack_kv_cache_varlen(d: Dims, hi, keep, ctx_lens, k: torch.Tensor, v: torch.Tensor,
                         cache: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Cache of a batch whose sequence b holds ctx_lens[b] tokens (version 3)."""
    b, hk, hd, n = d.batch, d.n_kv_heads, d.head_dim, d.seq_len
    _require(k, torch.bfloat16, (b, hk, n, hd), "k")
    _require(v, torch.bfloat16, (b, hk, n, hd), "v")
    hi, keep, cl = _i32(hi), _i32(keep), _cu(ctx_lens)
    if len(cl) != b:
        raise ValueError(f"ctx_lens: expected {b} lengths, got {len(cl)}")
    nbytes = kv_cache_bytes_varlen(d, hi, keep, cl)
    if cache is None:
        cache = torch.empty(nbytes, dtype=torch.uint8, device=k.device)
    check(_lib.lib.tria_pack_kv_cache_varlen(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi), cl.ctypes.data,
                                             _ptr(k), _ptr(v), _ptr(cache), cache.numel(), _stream(k.device)))
    return cache


def check_cache(d: Dims, cache: torch.Tensor, ctx_len: int) -> None:
    check(_lib.lib.tria_check_cache(C.byref(d), _ptr(cache), cache.numel(), ctx_len))


# ------------------------------------------------------------------ (5) decode
def decode_workspace_bytes(d: Dims, ctx_len: int) -> int:
    out = C.c_size_t(0)
    check(_lib.lib.tria_decode_workspace_bytes(C.byref(d), ctx_len, C.byref(out)))
    return out.value


def decode(d: Dims, cache: torch.Tensor, ctx_len: int, q: torch.Tensor, sm_scale: float,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    b, hq, hd = d.batch, d.n_q_heads, d.head_dim
    _require(q, torch.bfloat16, (b, hq, hd), "q")
    if out is None:
        out = torch.empty((b, hq, hd), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(d, ctx_len), dtype=torch.uint8, device=q.device)
    check(_lib.lib.tria_decode(C.byref(d), _ptr(cache), cache.numel(), ctx_len, _ptr(q), float(sm_scale),
                               _ptr(out), _ptr(workspace), workspace.numel(), _stream(q.device)))
    return out


def decode_noalloc(d: Dims, cache: torch.Tensor, ctx_len: int, q: torch.Tensor, sm_scale: float,
                   out: torch.Tensor) -> torch.Tensor:
    """decode with the library's own scratch (tria_decode_noalloc): no workspace, and
    nothing allocated here either (the caller passes out)."""
    b, hq, hd = d.batch, d.n_q_heads, d.head_dim
    _require(q, torch.bfloat16, (b, hq, hd), "q")
    _require(out, torch.float32, (b, hq, hd), "out")
    check(_lib.lib.tria_decode_noalloc(C.byref(d), _ptr(cache), cache.numel(), ctx_len, _ptr(q), float(sm_scale),
                                       _ptr(out), _stream(q.device)))
    return out


def decode_varlen(d: Dims, cache: torch.Tensor, q: torch.Tensor, sm_scale: float,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode over a pack_kv_cache_varlen cache: each sequence at its own length."""
    b, hq, hd = d.batch, d.n_q_heads, d.head_dim
    _require(q, torch.bfloat16, (b, hq, hd), "q")
    if out is None:
        out = torch.empty((b, hq, hd), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(d, d.seq_len), dtype=torch.uint8, device=q.device)
    check(_lib.lib.tria_decode_varlen(C.byref(d), _ptr(cache), cache.numel(), _ptr(q), float(sm_scale), _ptr(out),
                                      _ptr(workspace), workspace.numel(), _stream(q.device)))
    return out


# ------------------------------------------------------------------ paged cache
def paged_page_bytes(d: Dims) -> int:
    out = C.c_size_t(0)
    check(_lib.lib.tria_paged_page_bytes(C.byref(d), C.byref(out)))
    return out.value


def paged_table_bytes(d: Dims, ctx_len: int) -> int:
    out = C.c_size_t(0)
    check(_lib.lib.tria_paged_table_bytes(C.byref(d), ctx_len, C.byref(out)))
    return out.value


def build_paged_table(d: Dims, hi, keep, ctx_len, n_pages: int, free_pages,
                      old_table: Optional[np.ndarray] = None, seq_ids=None):
    """Host page table (uint8); returns (table, pages taken from the front of free_pages,
    released pages).  ctx_len: one length, or one per batch element (a variable-length
    table, tria_build_paged_table_varlen, where seq_ids optionally names the sequence
    of each slot: a slot whose id changed holds a new sequence)."""
    hi, keep = _i32(hi), _i32(keep)
    fp = _i32(free_pages)
    lens = None if np.isscalar(ctx_len) else np.ascontiguousarray(np.asarray(ctx_len, dtype=np.int64))
    table = np.zeros(paged_table_bytes(d, int(ctx_len) if lens is None else int(lens.max())), np.uint8)
    ot = None if old_table is None else np.ascontiguousarray(old_table, dtype=np.uint8)
    cap = 1 << 20 if ot is None else max(1, ot.size // 4)
    rel = np.zeros(cap, np.int32)
    used, nrel = C.c_int32(0), C.c_int32(0)
    common = (None if ot is None else ot.ctypes.data, 0 if ot is None else ot.size,
              fp.ctypes.data if fp.size else None, fp.size, table.ctypes.data, table.size, C.byref(used),
              rel.ctypes.data, cap, C.byref(nrel))
    if lens is None:
        check(_lib.lib.tria_build_paged_table(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi), ctx_len, n_pages,
                                              *common))
    else:
        sids = None if seq_ids is None else np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        if sids is not None and sids.shape != lens.shape:
            raise ValueError("seq_ids: one id per batch element")
        check(_lib.lib.tria_build_paged_table_varlen(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi),
                                                     lens.ctypes.data, None if sids is None else sids.ctypes.data,
                                                     n_pages, *common))
    return table, used.value, rel[:nrel.value].copy()


def pack_kv_cache_paged(d: Dims, hi, keep, ctx_len, k: torch.Tensor, v: torch.Tensor, table: torch.Tensor,
                        pool: torch.Tensor, old_table: Optional[torch.Tensor] = None) -> None:
    """Writes the records of `table` (device copy of build_paged_table's result) into pool.
    ctx_len: one length, or one per batch element (variable-length table)."""
    hi, keep = _i32(hi), _i32(keep)
    ot = (_ptr(old_table), 0 if old_table is None else old_table.numel())
    if np.isscalar(ctx_len):
        check(_lib.lib.tria_pack_kv_cache_paged(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi), ctx_len,
                                                _ptr(k), _ptr(v), _ptr(table), table.numel(), *ot, _ptr(pool),
                                                pool.numel(), _stream(pool.device)))
    else:
        lens = np.ascontiguousarray(np.asarray(ctx_len, dtype=np.int64))
        check(_lib.lib.tria_pack_kv_cache_paged_varlen(C.byref(d), hi.ctypes.data, keep.ctypes.data, len(hi),
                                                       lens.ctypes.data, _ptr(k), _ptr(v), _ptr(table), table.numel(),
                                                       *ot, _ptr(pool), pool.numel(), _stream(pool.device)))


def decode_paged(d: Dims, table: torch.Tensor, pool: torch.Tensor, ctx_len: int, q: torch.Tensor, sm_scale: float,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    b, hq, hd = d.batch, d.n_q_heads, d.head_dim
    _require(q, torch.bfloat16, (b, hq, hd), "q")
    if out is None:
        out = torch.empty((b, hq, hd), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(decode_skip_workspace_bytes(d, ctx_len), dtype=torch.uint8, device=q.device)
    check(_lib.lib.tria_decode_paged(C.byref(d), _ptr(table), table.numel(), _ptr(pool), pool.numel(), ctx_len,
                                     _ptr(q), float(sm_scale), _ptr(out), _ptr(workspace), workspace.numel(),
                                     _stream(q.device)))
    return out


def build_block_summaries_paged(d: Dims, table: torch.Tensor, pool: torch.Tensor, ctx_len: int,
                                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Statistics index of a paged cache (same layout as build_block_summaries)."""
    if out is None:
        out = torch.zeros(block_summaries_bytes(d, ctx_len), dtype=torch.uint8, device=pool.device)
    check(_lib.lib.tria_build_block_summaries_paged(C.byref(d), _ptr(table), table.numel(), _ptr(pool), pool.numel(),
                                                    ctx_len, _ptr(out), out.numel(), _stream(pool.device)))
    return out


def decode_skip_paged(d: Dims, table: torch.Tensor, pool: torch.Tensor, ctx_len: int, summaries: torch.Tensor,
                      q: torch.Tensor, thresholds: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode_skip over a paged cache."""
    b, hq, hd = d.batch, d.n_q_heads, d.head_dim
    _require(q, torch.bfloat16, (b, hq, hd), "q")
    _require(thresholds, torch.float32, (b, hq), "thresholds")
    if out is None:
        out = torch.empty((b, hq, hd), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(decode_skip_workspace_bytes(d, ctx_len), dtype=torch.uint8, device=q.device)
    check(_lib.lib.tria_decode_skip_paged(C.byref(d), _ptr(table), table.numel(), _ptr(pool), pool.numel(), ctx_len,
                                          _ptr(summaries), summaries.numel(), _ptr(q), _ptr(thresholds),
                                          float(sm_scale), _ptr(out), _ptr(workspace), workspace.numel(),
                                          _stream(q.device)))
    return out


def build_block_summaries_varlen(d: Dims, cache: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Statistics index of a variable-length (version-3) cache, sized for d.seq_len."""
    if out is None:
        out = torch.zeros(block_summaries_bytes(d, d.seq_len), dtype=torch.uint8, device=cache.device)
    check(_lib.lib.tria_build_block_summaries_varlen(C.byref(d), _ptr(cache), cache.numel(), _ptr(out), out.numel(),
                                                     _stream(cache.device)))
    return out


def decode_skip_varlen(d: Dims, cache: torch.Tensor, summaries: torch.Tensor, q: torch.Tensor,
                       thresholds: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode_skip over a variable-length cache: each sequence at its own length."""
    b, hq, hd = d.batch, d.n_q_heads, d.head_dim
    _require(q, torch.bfloat16, (b, hq, hd), "q")
    _require(thresholds, torch.float32, (b, hq), "thresholds")
    if out is None:
        out = torch.empty((b, hq, hd), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(decode_skip_workspace_bytes(d, d.seq_len), dtype=torch.uint8, device=q.device)
    check(_lib.lib.tria_decode_skip_varlen(C.byref(d), _ptr(cache), cache.numel(), _ptr(summaries), summaries.numel(),
                                           _ptr(q), _ptr(thresholds), float(sm_scale), _ptr(out), _ptr(workspace),
                                           workspace.numel(), _stream(q.device)))
    return out


def build_block_summaries_paged_varlen(d: Dims, table: torch.Tensor, pool: torch.Tensor,
                                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Statistics index of a variable-length paged cache, sized for d.seq_len."""
    if out is None:
        out = torch.zeros(block_summaries_bytes(d, d.seq_len), dtype=torch.uint8, device=pool.device)
    check(_lib.lib.tria_build_block_summaries_paged_varlen(C.byref(d), _ptr(table), table.numel(), _ptr(pool),
                                                           pool.numel(), _ptr(out), out.numel(), _stream(pool.device)))
    return out


def decode_skip_paged_varlen(d: Dims, table: torch.Tensor, pool: torch.Tensor, summaries: torch.Tensor,
                             q: torch.Tensor, thresholds: torch.Tensor, sm_scale: float,
                             out: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode_skip over a variable-length paged cache."""
    b, hq, hd = d.batch, d.n_q_heads, d.head_dim
    _require(q, torch.bfloat16, (b, hq, hd), "q")
    _require(thresholds, torch.float32, (b, hq), "thresholds")
    if out is None:
        out = torch.empty((b, hq, hd), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(decode_skip_workspace_bytes(d, d.seq_len), dtype=torch.uint8, device=q.device)
    check(_lib.lib.tria_decode_skip_paged_varlen(C.byref(d), _ptr(table), table.numel(), _ptr(pool), pool.numel(),
                                                 _ptr(summaries), summaries.numel(), _ptr(q), _ptr(thresholds),
                                                 float(sm_scale), _ptr(out), _ptr(workspace), workspace.numel(),
                                                 _stream(q.device)))
    return out


def decode_paged_varlen(d: Dims, table: torch.Tensor, pool: torch.Tensor, q: torch.Tensor, sm_scale: float,
                        out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode over a variable-length paged cache: each sequence at its own length."""
    b, hq, hd = d.batch, d.n_q_heads, d.head_dim
    _require(q, torch.bfloat16, (b, hq, hd), "q")
    if out is None:
        out = torch.empty((b, hq, hd), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(decode_skip_workspace_bytes(d, d.seq_len), dtype=torch.uint8, device=q.device)
    check(_lib.lib.tria_decode_paged_varlen(C.byref(d), _ptr(table), table.numel(), _ptr(pool), pool.numel(),
                                            _ptr(q), float(sm_scale), _ptr(out), _ptr(workspace), workspace.numel(),
                                            _stream(q.device)))
    return out


# ------------------------------------------------------------------ dynamic block skipping
def block_summaries_bytes(d: Dims, ctx_len: int) -> int:
    out = C.c_size_t(0)
    check(_lib.lib.tria_block_summaries_bytes(C.byref(d), ctx_len, C.byref(out)))
    return out.value


def build_block_summaries(d: Dims, cache: torch.Tensor, ctx_len: int,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Statistics index of a cache (uint8 device buffer, tria_block_summaries_bytes)."""
    if out is None:
        out = torch.zeros(block_summaries_bytes(d, ctx_len), dtype=torch.uint8, device=cache.device)
    check(_lib.lib.tria_build_block_summaries(C.byref(d), _ptr(cache), cache.numel(), ctx_len, _ptr(out), out.numel(),
                                              _stream(cache.device)))
    return out


def skip_masks(d: Dims, cache: torch.Tensor, ctx_len: int, summaries: torch.Tensor, q: torch.Tensor,
               thresholds: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Keep bits per stored record: int32 view of uint32 [batch * n_kv_heads][rmax]."""
    b, hq, hd = d.batch, d.n_q_heads, d.head_dim
    _require(q, torch.bfloat16, (b, hq, hd), "q")
    _require(thresholds, torch.float32, (b, hq), "thresholds")
    rmax = (ctx_len - 1) // d.block + 1
    if out is None:
        out = torch.zeros((b * d.n_kv_heads, rmax), dtype=torch.int32, device=q.device)
    check(_lib.lib.tria_skip_masks(C.byref(d), _ptr(cache), cache.numel(), ctx_len, _ptr(summaries),
                                   summaries.numel(), _ptr(q), _ptr(thresholds), float(sm_scale), _ptr(out),
                                   out.numel() * 4, _stream(q.device)))
    return out


def decode_skip_workspace_bytes(d: Dims, ctx_len: int) -> int:
    out = C.c_size_t(0)
    check(_lib.lib.tria_decode_skip_workspace_bytes(C.byref(d), ctx_len, C.byref(out)))
    return out.value


def decode_skip(d: Dims, cache: torch.Tensor, ctx_len: int, summaries: torch.Tensor, q: torch.Tensor,
                thresholds: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode reading only the records some query head keeps (fp32 [b][Hq][d])."""
    b, hq, hd = d.batch, d.n_q_heads, d.head_dim
    _require(q, torch.bfloat16, (b, hq, hd), "q")
    _require(thresholds, torch.float32, (b, hq), "thresholds")
    if out is None:
        out = torch.empty((b, hq, hd), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(decode_skip_workspace_bytes(d, ctx_len), dtype=torch.uint8, device=q.device)
    check(_lib.lib.tria_decode_skip(C.byref(d), _ptr(cache), cache.numel(), ctx_len, _ptr(summaries),
                                    summaries.numel(), _ptr(q), _ptr(thresholds), float(sm_scale), _ptr(out),
                                    _ptr(workspace), workspace.numel(), _stream(q.device)))
    return out


# ------------------------------------------------------------------ calibration
def policy_cost(d: Dims, hi: int, keep: int, cost_int8: float = 1.0, cost_int4: float = 1.0) -> float:
    """Cost of one head's (hi, keep): whole kept tiles x block^2, weighted per precision."""
    out = C.c_double(0.0)
    check(_lib.lib.tria_policy_cost(C.byref(d), int(hi), int(keep), float(cost_int8), float(cost_int4),
                                    C.byref(out)))
    return out.value


def allocate_policy(d: Dims, err: np.ndarray, budget: float, cost_int8: float = 1.0, cost_int4: float = 1.0):
    """Greedy per-head (hi, keep) under a cost budget from error tables err[h][hi][keep]
    (shape (n_heads, K + 1, K + 1)); returns (hi, keep, total_cost, total_err)."""
    err = np.ascontiguousarray(np.asarray(err, dtype=np.float64))
    if err.ndim != 3 or err.shape[1] != err.shape[2]:
        raise ValueError(f"err: expected (n_heads, K + 1, K + 1), got {err.shape}")
    n_heads, K = err.shape[0], err.shape[1] - 1
    hi = np.zeros(n_heads, np.int32)
    keep = np.zeros(n_heads, np.int32)
    tc, te = C.c_double(0.0), C.c_double(0.0)
    check(_lib.lib.tria_allocate_policy(C.byref(d), n_heads, K, err.ctypes.data, float(cost_int8), float(cost_int4),
                                        float(budget), hi.ctypes.data, keep.ctypes.data, C.byref(tc), C.byref(te)))
    return hi, keep, tc.value, te.value


# ------------------------------------------------------------------ measured ceilings
def peak_mfma(kind: int, iters: int, sink: torch.Tensor) -> float:
    """Enqueues the MFMA issue loop (kind 0: int8 16x16x64, 1: bf16 16x16x32) on the
    current stream of sink's device; returns the int8 ops (bf16 flops) of the launch."""
    _require(sink, torch.int32, (_lib.PEAK_SINK_INTS,), "sink")
    work = C.c_double(0.0)
    check(_lib.lib.tria_peak_mfma(int(kind), int(iters), _ptr(sink), C.byref(work), _stream(sink.device)))
    return work.value


def peak_read(src: torch.Tensor, sink: torch.Tensor) -> float:
    """Enqueues the streaming read of all of src (uint8, a multiple of 64 MiB) on the
    current stream of its device; returns the bytes read."""
    _require(src, torch.uint8, (src.numel(),), "src")
    _require(sink, torch.int32, (_lib.PEAK_SINK_INTS,), "sink")
    work = C.c_double(0.0)
    check(_lib.lib.tria_peak_read(_ptr(src), src.numel(), _ptr(sink), C.byref(work), _stream(src.device)))
    return work.value
