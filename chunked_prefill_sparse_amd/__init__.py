"""CompactAttention chunked-prefill hot path for MI355X (gfx950).

Thin Python binding over the C ABI of ``libcompact_attn.so``
(``include/compact_attn.h``): argument checks and marshalling only.  Every
step of the path runs in the library's HIP kernels; torch supplies device
memory and the current stream.

    T, lens = build_union_tables(mask, H_kv, n_q_blocks, n_kv_blocks)
    O       = chunk_attention(q, k_cache, v_cache, T, lens, prior_len, chunk_len)

Selection (Block-Union KV tables) and execution (zero-copy paged attention over
a KV-head-major cache) are separate calls, as in the method.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import CA_BLOCK, CA_MAX_BATCH, CompactAttnError  # noqa: F401

__all__ = ["build_union_tables", "chunk_attention", "tables_to_csr", "check_tables",
           "build_union_tables_devlen", "chunk_attention_devlen", "chunk_attention_stamped",
           "stamps_summary",
           "compact_kv", "append_kv",
           "build_row_tables", "chunk_attention_rows", "pool_blocks", "block_mask_topk", "select_chunk",
           "append_select_chunk",
           "workspace_size", "balanced_workspace_size", "chunk_attention_split_noalloc",
           "CompactAttnError", "library_path"]


def library_path() -> str:
    return _lib.LIB_PATH


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _need_cuda(name: str, t: torch.Tensor, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda) tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _host_ints(name: str, vals: Sequence[int], B: int):
    vals = [int(v) for v in (vals.tolist() if hasattr(vals, "tolist") else vals)]
    if len(vals) != B:
        raise ValueError(f"{name} must have {B} entries")
    return _lib.int_array(vals)


def build_union_tables(mask: torch.Tensor, H_kv: int, n_q_blocks: Sequence[int],
                       n_kv_blocks: Sequence[int], T: Optional[torch.Tensor] = None,
                       lens: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None
                       ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Block-Union KV selection: mask uint8 [B, H_q, NQ_max, NKB_max] (device) ->
    (T int32 [B, H_kv, NKB_max] ascending, -1 padded; lens int32 [B, H_kv])."""
    _need_cuda("mask", mask, torch.uint8)
    if mask.dim() != 4:
        raise ValueError("mask must be [B, H_q, NQ_max, NKB_max]")
    B, H_q, NQ_max, NKB_max = mask.shape
    if H_kv < 1 or H_q % H_kv:
        raise ValueError("H_q must be a positive multiple of H_kv")
    if T is None:
        T = torch.empty((B, H_kv, NKB_max), dtype=torch.int32, device=mask.device)
    if lens is None:
        lens = torch.empty((B, H_kv), dtype=torch.int32, device=mask.device)
    _need_cuda("T", T, torch.int32)
    _need_cuda("lens", lens, torch.int32)
    if tuple(T.shape) != (B, H_kv, NKB_max) or tuple(lens.shape) != (B, H_kv):
        raise ValueError("T / lens have the wrong shape")
    st = _lib.lib().ca_build_union_tables(
        mask.data_ptr(), B, H_q, H_kv, NQ_max, NKB_max, _host_ints("n_q_blocks", n_q_blocks, B),
        _host_ints("n_kv_blocks", n_kv_blocks, B), T.data_ptr(), lens.data_ptr(),
        _stream_ptr(stream))
    _lib.check(st, "ca_build_union_tables")
    return T, lens


def _dev_ints(name: str, t: torch.Tensor, B: int):
    _need_cuda(name, t, torch.int32)
    if t.dim() != 1 or t.shape[0] != B:
        raise ValueError(f"{name} must be a device int32 tensor of {B} entries")
    return t.data_ptr()


def build_union_tables_devlen(mask: torch.Tensor, H_kv: int, n_q_blocks: torch.Tensor,
                              n_kv_blocks: torch.Tensor, T: Optional[torch.Tensor] = None,
                              lens: Optional[torch.Tensor] = None,
                              stream: Optional[torch.cuda.Stream] = None
                              ) -> Tuple[torch.Tensor, torch.Tensor]:
    """``build_union_tables`` with the extents n_q_blocks / n_kv_blocks as device
    int32 [B] tensors, read by the kernel when it runs (graph replay with new
    extents)."""
    _need_cuda("mask", mask, torch.uint8)
    if mask.dim() != 4:
        raise ValueError("mask must be [B, H_q, NQ_max, NKB_max]")
    B, H_q, NQ_max, NKB_max = mask.shape
    if H_kv < 1 or H_q % H_kv:
        raise ValueError("H_q must be a positive multiple of H_kv")
    if T is None:
        T = torch.empty((B, H_kv, NKB_max), dtype=torch.int32, device=mask.device)
    if lens is None:
        lens = torch.empty((B, H_kv), dtype=torch.int32, device=mask.device)
    _need_cuda("T", T, torch.int32)
    _need_cuda("lens", lens, torch.int32)
    if tuple(T.shape) != (B, H_kv, NKB_max) or tuple(lens.shape) != (B, H_kv):
        raise ValueError("T / lens have the wrong shape")
    st = _lib.lib().ca_build_union_tables_devlen(
        mask.data_ptr(), B, H_q, H_kv, NQ_max, NKB_max, _dev_ints("n_q_blocks", n_q_blocks, B),
        _dev_ints("n_kv_blocks", n_kv_blocks, B), T.data_ptr(), lens.data_ptr(),
        _stream_ptr(stream))
    _lib.check(st, "ca_build_union_tables_devlen")
    return T, lens


def chunk_attention_devlen(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           T: torch.Tensor, lens: torch.Tensor, prior_len: torch.Tensor,
                           chunk_len: torch.Tensor, scale: Optional[float] = None,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                           return_lse: bool = False, stream: Optional[torch.cuda.Stream] = None):
    """``chunk_attention`` with prior_len / chunk_len as device int32 [B] tensors,
    read by the kernels when they run: one captured graph serves every chunk
    offset.  Lengths that break the call's limits give that sequence O = 0 and
    lse = -inf."""
    B, H_q, H_kv, C_max, L, D, scale, out, lse, dt = _attention_args(
        q, k_cache, v_cache, scale, out, lse, return_lse)
    _need_cuda("T", T, torch.int32)
    _need_cuda("lens", lens, torch.int32)
    if T.dim() != 3 or tuple(T.shape[:2]) != (B, H_kv) or tuple(lens.shape) != (B, H_kv):
        raise ValueError("T must be [B, H_kv, NKB_max] and lens [B, H_kv]")
    st = _lib.lib().ca_chunk_attention_devlen(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), T.data_ptr(), lens.data_ptr(),
        T.shape[2], _dev_ints("prior_len", prior_len, B), _dev_ints("chunk_len", chunk_len, B),
        B, H_q, H_kv, C_max, L, D, CA_BLOCK, scale, dt, out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream_ptr(stream))
    _lib.check(st, "ca_chunk_attention_devlen")
    return (out, lse) if return_lse else out


def check_tables(T: torch.Tensor, lens: torch.Tensor, n_kv_blocks: Sequence[int],
                 row_bad: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Contract check of tables (``ca_check_tables``): int32 [B, H_kv] (device),
    0 for a well-formed row, else a bitmask (1 length out of range, 2 entry
    out of range, 4 not strictly ascending, 8 padding other than -1)."""
    _need_cuda("T", T, torch.int32)
    _need_cuda("lens", lens, torch.int32)
    if T.dim() != 3 or lens.dim() != 2 or tuple(lens.shape) != tuple(T.shape[:2]):
        raise ValueError("T must be [B, H_kv, NKB_max] and lens [B, H_kv]")
    B, H_kv, NKB_max = T.shape
    if row_bad is None:
        row_bad = torch.empty((B, H_kv), dtype=torch.int32, device=T.device)
    _need_cuda("row_bad", row_bad, torch.int32)
    if tuple(row_bad.shape) != (B, H_kv):
        raise ValueError("row_bad must be [B, H_kv]")
    st = _lib.lib().ca_check_tables(T.data_ptr(), lens.data_ptr(), B, H_kv, NKB_max,
                                    _host_ints("n_kv_blocks", n_kv_blocks, B),
                                    row_bad.data_ptr(), _stream_ptr(stream))
    _lib.check(st, "ca_check_tables")
    return row_bad


def build_row_tables(mask: torch.Tensor, n_kv_blocks: Sequence[int],
                     T: Optional[torch.Tensor] = None, lens: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None
                     ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-(head, Q-block) block lists of a block-sparse kernel (no union):
    mask uint8 [B, H_q, NQ_max, NKB_max] -> (T_rows int32 [B, H_q, NQ_max, NKB_max]
    ascending, -1 padded; lens int32 [B, H_q, NQ_max]).  The union builder on the
    mask viewed as one-row groups."""
    _need_cuda("mask", mask, torch.uint8)
    if mask.dim() != 4:
        raise ValueError("mask must be [B, H_q, NQ_max, NKB_max]")
    B, H_q, NQ_max, NKB_max = mask.shape
    rows = mask.view(B, H_q * NQ_max, 1, NKB_max)
    if T is not None:
        T = T.view(B, H_q * NQ_max, NKB_max)
    if lens is not None:
        lens = lens.view(B, H_q * NQ_max)
    T, lens = build_union_tables(rows, H_q * NQ_max, [1] * B, n_kv_blocks, T, lens, stream)
    return T.view(B, H_q, NQ_max, NKB_max), lens.view(B, H_q, NQ_max)


def _attention_args(q, k_cache, v_cache, scale, out, lse, return_lse):
    _need_cuda("q", q)
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be bfloat16 or float32")
    _need_cuda("k_cache", k_cache, q.dtype)
    _need_cuda("v_cache", v_cache, q.dtype)
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B,H_q,C_max,D], caches [B,H_kv,L,D]")
    B, H_q, C_max, D = q.shape
    Bk, H_kv, L, Dk = k_cache.shape
    if Bk != B or Dk != D:
        raise ValueError("cache batch / head dim do not match q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _need_cuda("out", out, q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if return_lse and lse is None:
        lse = torch.empty((B, H_q, C_max), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need_cuda("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, H_q, C_max):
            raise ValueError("lse must be [B, H_q, C_max]")
    dt = _lib.CA_BF16 if q.dtype == torch.bfloat16 else _lib.CA_F32
    return B, H_q, H_kv, C_max, L, D, float(scale), out, lse, dt


def chunk_attention_rows(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         T_rows: torch.Tensor, lens_rows: torch.Tensor, prior_len: Sequence[int],
                         chunk_len: Sequence[int], scale: Optional[float] = None,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         return_lse: bool = False, stream: Optional[torch.cuda.Stream] = None):
    """Block-sparse-kernel execution (the baseline the union replaces): each
    64-row Q-block of each head attends the blocks of its own list
    T_rows[b, h, qb] (from ``build_row_tables``)."""
    B, H_q, H_kv, C_max, L, D, scale, out, lse, dt = _attention_args(
        q, k_cache, v_cache, scale, out, lse, return_lse)
    _need_cuda("T_rows", T_rows, torch.int32)
    _need_cuda("lens_rows", lens_rows, torch.int32)
    if T_rows.dim() != 4 or tuple(T_rows.shape[:2]) != (B, H_q) or \
            tuple(lens_rows.shape) != tuple(T_rows.shape[:3]):
        raise ValueError("T_rows must be [B, H_q, NQ_max, NKB_max] and lens_rows [B, H_q, NQ_max]")
    NQ_max, NKB_max = T_rows.shape[2], T_rows.shape[3]
    st = _lib.lib().ca_chunk_attention_rows(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), T_rows.data_ptr(),
        lens_rows.data_ptr(), NQ_max, NKB_max, _host_ints("prior_len", prior_len, B),
        _host_ints("chunk_len", chunk_len, B), B, H_q, H_kv, C_max, L, D, CA_BLOCK, scale, dt,
        out.data_ptr(), lse.data_ptr() if lse is not None else None, _stream_ptr(stream))
    _lib.check(st, "ca_chunk_attention_rows")
    return (out, lse) if return_lse else out


def workspace_size(B: int, H_q: int, C_max: int, D: int, n_splits: int) -> int:
    """Bytes of workspace ``chunk_attention(..., n_splits=n)`` needs (0 for n < 2)."""
    return int(_lib.lib().ca_chunk_attention_workspace_size(B, H_q, C_max, D, n_splits))


def balanced_workspace_size(B: int, H_q: int, H_kv: int, C_max: int, D: int) -> int:
    """Bytes of workspace ``chunk_attention(..., balanced=True)`` needs."""
    return int(_lib.lib().ca_chunk_attention_balanced_workspace_size(B, H_q, H_kv, C_max, D))


def chunk_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    T: torch.Tensor, lens: torch.Tensor, prior_len: Sequence[int],
                    chunk_len: Sequence[int], scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    return_lse: bool = False, stream: Optional[torch.cuda.Stream] = None,
                    n_splits: int = 1, workspace: Optional[torch.Tensor] = None,
                    balanced: bool = False):
    """Zero-copy paged chunk attention.

    q [B, H_q, C_max, D] and k_cache/v_cache [B, H_kv, L, D] (bf16 or fp32, device);
    T/lens from ``build_union_tables``; prior_len/chunk_len host ints per sequence.
    Returns O [B, H_q, C_max, D] (and lse fp32 [B, H_q, C_max] if ``return_lse``).
    ``n_splits`` > 1 (bf16 or fp32) cuts each table into that many ranges run by separate
    workgroups and merged (``ca_chunk_attention_split``); ``workspace`` is then a
    device tensor of at least ``workspace_size(...)`` bytes (allocated if None).
    ``balanced`` plans the work on the device so that uneven tables spread evenly over
    the compute units (``ca_chunk_attention_balanced``); ``workspace`` is then at least
    ``balanced_workspace_size(...)`` bytes (allocated if None).
    """
    _need_cuda("q", q)
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be bfloat16 or float32")
    _need_cuda("k_cache", k_cache, q.dtype)
    _need_cuda("v_cache", v_cache, q.dtype)
    _need_cuda("T", T, torch.int32)
    _need_cuda("lens", lens, torch.int32)
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B,H_q,C_max,D], caches [B,H_kv,L,D]")
    B, H_q, C_max, D = q.shape
    Bk, H_kv, L, Dk = k_cache.shape
    if Bk != B or Dk != D:
        raise ValueError("cache batch / head dim do not match q")
    if T.dim() != 3 or tuple(T.shape[:2]) != (B, H_kv) or tuple(lens.shape) != (B, H_kv):
        raise ValueError("T must be [B, H_kv, NKB_max] and lens [B, H_kv]")
    NKB_max = T.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _need_cuda("out", out, q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if return_lse and lse is None:
        lse = torch.empty((B, H_q, C_max), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need_cuda("lse", lse, torch.float32)
        if tuple(lse.shape) != (B, H_q, C_max):
            raise ValueError("lse must be [B, H_q, C_max]")
    dt = _lib.CA_BF16 if q.dtype == torch.bfloat16 else _lib.CA_F32
    if balanced and n_splits > 1:
        raise ValueError("balanced and n_splits > 1 are exclusive")
    if balanced:
        need = balanced_workspace_size(B, H_q, H_kv, C_max, D)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _need_cuda("workspace", workspace)
        wbytes = workspace.numel() * workspace.element_size()
        st = _lib.lib().ca_chunk_attention_balanced(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), T.data_ptr(), lens.data_ptr(),
            NKB_max, _host_ints("prior_len", prior_len, B), _host_ints("chunk_len", chunk_len, B),
            B, H_q, H_kv, C_max, L, D, CA_BLOCK, float(scale), dt, workspace.data_ptr(), wbytes,
            out.data_ptr(), lse.data_ptr() if lse is not None else None, _stream_ptr(stream))
        _lib.check(st, "ca_chunk_attention_balanced")
        return (out, lse) if return_lse else out
    if n_splits > 1:
        need = workspace_size(B, H_q, C_max, D, n_splits)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _need_cuda("workspace", workspace)
        wbytes = workspace.numel() * workspace.element_size()
        st = _lib.lib().ca_chunk_attention_split(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), T.data_ptr(), lens.data_ptr(),
            NKB_max, _host_ints("prior_len", prior_len, B), _host_ints("chunk_len", chunk_len, B),
            B, H_q, H_kv, C_max, L, D, CA_BLOCK, float(scale), dt, int(n_splits),
            workspace.data_ptr(), wbytes, out.data_ptr(),
            lse.data_ptr() if lse is not None else None, _stream_ptr(stream))
        _lib.check(st, "ca_chunk_attention_split")
        return (out, lse) if return_lse else out
    st = _lib.lib().ca_chunk_attention(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), T.data_ptr(), lens.data_ptr(),
        NKB_max, _host_ints("prior_len", prior_len, B), _host_ints("chunk_len", chunk_len, B),
        B, H_q, H_kv, C_max, L, D, CA_BLOCK, float(scale), dt, out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream_ptr(stream))
    _lib.check(st, "ca_chunk_attention")
    return (out, lse) if return_lse else out


def chunk_attention_split_noalloc(q: torch.Tensor, k_cache: torch.Tensor,
                                  v_cache: torch.Tensor, T: torch.Tensor, lens: torch.Tensor,
                                  prior_len: Sequence[int], chunk_len: Sequence[int],
                                  n_splits: int, scale: Optional[float] = None,
                                  out: Optional[torch.Tensor] = None,
                                  lse: Optional[torch.Tensor] = None, return_lse: bool = False,
                                  stream: Optional[torch.cuda.Stream] = None):
    """Split-KV chunk attention whose partials live in the library's static device
    array (``ca_chunk_attention_split_noalloc``): the library allocates nothing.
    Pass ``out`` (and ``lse``) to allocate nothing here either.  Calls that
    overlap on one device race on the shared array."""
    B, H_q, H_kv, C_max, L, D, scale, out, lse, dt = _attention_args(
        q, k_cache, v_cache, scale, out, lse, return_lse)
    _need_cuda("T", T, torch.int32)
    _need_cuda("lens", lens, torch.int32)
    if T.dim() != 3 or tuple(T.shape[:2]) != (B, H_kv) or tuple(lens.shape) != (B, H_kv):
        raise ValueError("T must be [B, H_kv, NKB_max] and lens [B, H_kv]")
    st = _lib.lib().ca_chunk_attention_split_noalloc(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), T.data_ptr(), lens.data_ptr(),
        T.shape[2], _host_ints("prior_len", prior_len, B), _host_ints("chunk_len", chunk_len, B),
        B, H_q, H_kv, C_max, L, D, CA_BLOCK, scale, dt, int(n_splits), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream_ptr(stream))
    _lib.check(st, "ca_chunk_attention_split_noalloc")
    return (out, lse) if return_lse else out


def chunk_attention_stamped(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            T: torch.Tensor, lens: torch.Tensor, prior_len: Sequence[int],
                            chunk_len: Sequence[int], scale: Optional[float] = None,
                            out: Optional[torch.Tensor] = None,
                            stamps: Optional[torch.Tensor] = None,
                            stream: Optional[torch.cuda.Stream] = None):
    """``chunk_attention`` (bf16) that also records per-workgroup timing words
    (``ca_chunk_attention_stamped``).  Returns (O, stamps int32 [n_wg, 4]);
    ``stamps_summary`` turns them into durations and the shader clock."""
    B, H_q, H_kv, C_max, L, D, scale, out, _, dt = _attention_args(
        q, k_cache, v_cache, scale, out, None, False)
    _need_cuda("T", T, torch.int32)
    _need_cuda("lens", lens, torch.int32)
    if T.dim() != 3 or tuple(T.shape[:2]) != (B, H_kv) or tuple(lens.shape) != (B, H_kv):
        raise ValueError("T must be [B, H_kv, NKB_max] and lens [B, H_kv]")
    n = ctypes.c_int(0)
    for _ in range(2):  # a first call without a large enough buffer reports the count
        cap = 0 if stamps is None else stamps.numel() // 4
        st = _lib.lib().ca_chunk_attention_stamped(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), T.data_ptr(), lens.data_ptr(),
            T.shape[2], _host_ints("prior_len", prior_len, B),
            _host_ints("chunk_len", chunk_len, B), B, H_q, H_kv, C_max, L, D, CA_BLOCK, scale,
            dt, out.data_ptr(), None, 0 if stamps is None else stamps.data_ptr(), cap,
            ctypes.byref(n), _stream_ptr(stream))
        if st == _lib.CA_OK:
            return out, stamps[:n.value]
        if stamps is not None and n.value <= cap:
            break
        stamps = torch.zeros((max(n.value, 1), 4), dtype=torch.int32, device=q.device)
    _lib.check(st, "ca_chunk_attention_stamped")


def stamps_summary(stamps: torch.Tensor) -> dict:
    """Durations (us) and shader clock (GHz) from ``chunk_attention_stamped``'s
    records: overall, and the clock per XCC."""
    import numpy as np
    a = stamps.cpu().numpy().view(np.uint32).astype(np.float64)
    ticks, cycles = a[:, 1], a[:, 2]
    xcc = (a[:, 3].astype(np.int64) & 0xF)
    ghz = cycles / np.maximum(ticks, 1) * 0.1
    per = {int(x): round(float(ghz[xcc == x].mean()), 4) for x in np.unique(xcc)}
    start = a[:, 0]
    span_us = float(((start + ticks).max() - start.min()) / 100.0)
    return dict(workgroups=int(a.shape[0]), clock_GHz=round(float(cycles.sum() / ticks.sum() * 0.1), 4),
                clock_GHz_by_xcc=per, wg_us_mean=round(float(ticks.mean() / 100.0), 2),
                wg_us_max=round(float(ticks.max() / 100.0), 2), span_us=round(span_us, 2),
                cycles_per_wg_mean=round(float(cycles.mean()), 1))


def tables_to_csr(T: torch.Tensor, lens: torch.Tensor, L: int,
                  stream: Optional[torch.cuda.Stream] = None):
    """Paged-metadata view: (kv_indptr int32 [B*H_kv+1], kv_indices int32
    [B*H_kv*NKB_max], of which the first kv_indptr[-1] entries are valid)."""
    _need_cuda("T", T, torch.int32)
    _need_cuda("lens", lens, torch.int32)
    B, H_kv, NKB_max = T.shape
    indptr = torch.empty(B * H_kv + 1, dtype=torch.int32, device=T.device)
    indices = torch.empty(B * H_kv * NKB_max, dtype=torch.int32, device=T.device)
    st = _lib.lib().ca_tables_to_csr(T.data_ptr(), lens.data_ptr(), B, H_kv, NKB_max, int(L),
                                     indptr.data_ptr(), indices.data_ptr(), _stream_ptr(stream))
    _lib.check(st, "ca_tables_to_csr")
    return indptr, indices


def append_kv(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
              v_cache: torch.Tensor, prior_len: Sequence[int], chunk_len: Sequence[int],
              stream: Optional[torch.cuda.Stream] = None) -> None:
    """Write a chunk's keys and values (k_new, v_new [B, H_kv, C_max, D], rows
    [0, chunk_len[b]) used) into the caches [B, H_kv, L, D] at rows
    [prior_len[b], prior_len[b] + chunk_len[b]) (``ca_append_kv``)."""
    _need_cuda("k_new", k_new)
    if k_new.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("k_new must be bfloat16 or float32")
    for name, t in (("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _need_cuda(name, t, k_new.dtype)
    if k_new.dim() != 4 or v_new.shape != k_new.shape or k_cache.dim() != 4 or \
            v_cache.shape != k_cache.shape:
        raise ValueError("k_new/v_new must be [B, H_kv, C_max, D] and the caches [B, H_kv, L, D]")
    B, H_kv, C_max, D = k_new.shape
    if tuple(k_cache.shape[:2]) != (B, H_kv) or k_cache.shape[3] != D:
        raise ValueError("cache batch / heads / head dim do not match the new rows")
    dt = _lib.CA_BF16 if k_new.dtype == torch.bfloat16 else _lib.CA_F32
    st = _lib.lib().ca_append_kv(k_new.data_ptr(), v_new.data_ptr(), B, H_kv, C_max,
                                 k_cache.shape[2], D, dt, _host_ints("prior_len", prior_len, B),
                                 _host_ints("chunk_len", chunk_len, B), k_cache.data_ptr(),
                                 v_cache.data_ptr(), _stream_ptr(stream))
    _lib.check(st, "ca_append_kv")


def compact_kv(k_cache: torch.Tensor, v_cache: torch.Tensor, T: torch.Tensor,
               lens: torch.Tensor, prior_len: Sequence[int], chunk_len: Sequence[int],
               k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None,
               T_out: Optional[torch.Tensor] = None,
               stream: Optional[torch.cuda.Stream] = None):
    """Explicit KV compaction (the copy that zero-copy execution avoids).

    Copies the selected prior blocks of each (b, g) into contiguous blocks that
    end where the chunk starts, keeps chunk blocks in place, and returns
    (k_out, v_out, T_out) such that ``chunk_attention(q, k_out, v_out, T_out,
    lens, ...)`` equals ``chunk_attention(q, k_cache, v_cache, T, lens, ...)``.
    Blocks of k_out/v_out that no table entry lands on are left unwritten.
    """
    _need_cuda("k_cache", k_cache)
    if k_cache.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("k_cache must be bfloat16 or float32")
    _need_cuda("v_cache", v_cache, k_cache.dtype)
    _need_cuda("T", T, torch.int32)
    _need_cuda("lens", lens, torch.int32)
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, H_kv, L, D] and alike")
    B, H_kv, L, D = k_cache.shape
    if T.dim() != 3 or tuple(T.shape[:2]) != (B, H_kv) or tuple(lens.shape) != (B, H_kv):
        raise ValueError("T must be [B, H_kv, NKB_max] and lens [B, H_kv]")
    NKB_max = T.shape[2]
    if k_out is None:
        k_out = torch.empty_like(k_cache)
    if v_out is None:
        v_out = torch.empty_like(v_cache)
    if T_out is None:
        T_out = torch.empty_like(T)
    _need_cuda("k_out", k_out, k_cache.dtype)
    _need_cuda("v_out", v_out, k_cache.dtype)
    _need_cuda("T_out", T_out, torch.int32)
    if k_out.shape != k_cache.shape or v_out.shape != k_cache.shape or T_out.shape != T.shape:
        raise ValueError("outputs must have the shapes of the caches and of T")
    dt = _lib.CA_BF16 if k_cache.dtype == torch.bfloat16 else _lib.CA_F32
    st = _lib.lib().ca_compact_kv(
        k_cache.data_ptr(), v_cache.data_ptr(), T.data_ptr(), lens.data_ptr(), NKB_max,
        _host_ints("prior_len", prior_len, B), _host_ints("chunk_len", chunk_len, B), B, H_kv,
        L, D, dt, k_out.data_ptr(), v_out.data_ptr(), T_out.data_ptr(), _stream_ptr(stream))
    _lib.check(st, "ca_compact_kv")
    return k_out, v_out, T_out


def pool_blocks(x: torch.Tensor, blk_begin: Sequence[int], blk_end: Sequence[int],
                out: Optional[torch.Tensor] = None, n_out: Optional[int] = None,
                stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Mean of each 64-row block: x [B, H, R, D] (bf16/fp32) -> out float32
    [B, H, n_out, D], entries blk_begin[b] <= kb < blk_end[b] written, the rest
    left as they were (a new ``out`` starts as zeros)."""
    _need_cuda("x", x)
    if x.dtype not in (torch.bfloat16, torch.float32) or x.dim() != 4:
        raise ValueError("x must be a bfloat16/float32 [B, H, R, D] tensor")
    B, H, R, D = x.shape
    if out is None:
        out = torch.zeros((B, H, n_out if n_out is not None else R // CA_BLOCK, D),
                          dtype=torch.float32, device=x.device)
    _need_cuda("out", out, torch.float32)
    if out.dim() != 4 or tuple(out.shape[:2]) != (B, H) or out.shape[3] != D:
        raise ValueError("out must be [B, H, n_out, D]")
    dt = _lib.CA_BF16 if x.dtype == torch.bfloat16 else _lib.CA_F32
    st = _lib.lib().ca_pool_blocks(x.data_ptr(), dt, B, H, R, D,
                                   _host_ints("blk_begin", blk_begin, B),
                                   _host_ints("blk_end", blk_end, B), out.data_ptr(),
                                   out.shape[2], _stream_ptr(stream))
    _lib.check(st, "ca_pool_blocks")
    return out


def block_mask_topk(qbar: torch.Tensor, kbar: torch.Tensor, prior_len: Sequence[int],
                    chunk_len: Sequence[int], budget: int, local: int,
                    scores: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None):
    """Pooled block scores and the per-row top-k mask (sink, local window and
    causal block triangle always on).  qbar [B, H_q, NQ_max, D], kbar
    [B, H_kv, NKB_max, D] float32.  Returns (mask uint8 [B, H_q, NQ_max, NKB_max],
    scores float32 of the same shape)."""
    _need_cuda("qbar", qbar, torch.float32)
    _need_cuda("kbar", kbar, torch.float32)
    if qbar.dim() != 4 or kbar.dim() != 4 or qbar.shape[0] != kbar.shape[0] or \
            qbar.shape[3] != kbar.shape[3]:
        raise ValueError("qbar must be [B, H_q, NQ_max, D] and kbar [B, H_kv, NKB_max, D]")
    B, H_q, NQ_max, D = qbar.shape
    H_kv, NKB_max = kbar.shape[1], kbar.shape[2]
    shape = (B, H_q, NQ_max, NKB_max)
    if scores is None:
        scores = torch.empty(shape, dtype=torch.float32, device=qbar.device)
    if mask is None:
        mask = torch.empty(shape, dtype=torch.uint8, device=qbar.device)
    _need_cuda("scores", scores, torch.float32)
    _need_cuda("mask", mask, torch.uint8)
    if tuple(scores.shape) != shape or tuple(mask.shape) != shape:
        raise ValueError(f"scores and mask must be {shape}")
    st = _lib.lib().ca_block_mask_topk(
        qbar.data_ptr(), kbar.data_ptr(), B, H_q, H_kv, NQ_max, NKB_max, D,
        _host_ints("prior_len", prior_len, B), _host_ints("chunk_len", chunk_len, B),
        int(budget), int(local), scores.data_ptr(), mask.data_ptr(), _stream_ptr(stream))
    _lib.check(st, "ca_block_mask_topk")
    return mask, scores


def _select_lengths(fn: str, prior_len, chunk_len, B: int):
    """The selection calls take host sequences (``fn``) or device int32 [B]
    tensors (``fn``_devlen, read by the kernels when they run)."""
    dev = isinstance(prior_len, torch.Tensor) or isinstance(chunk_len, torch.Tensor)
    if not dev:
        return fn, _host_ints("prior_len", prior_len, B), _host_ints("chunk_len", chunk_len, B)
    if not (isinstance(prior_len, torch.Tensor) and isinstance(chunk_len, torch.Tensor)):
        raise ValueError("prior_len and chunk_len must both be host sequences or both device tensors")
    return (fn + "_devlen", _dev_ints("prior_len", prior_len, B),
            _dev_ints("chunk_len", chunk_len, B))


def select_chunk(q_chunk: torch.Tensor, k_cache: torch.Tensor, prior_len: Sequence[int],
                 chunk_len: Sequence[int], budget: int, local: int, qbar: torch.Tensor,
                 kbar: torch.Tensor, scores: torch.Tensor, mask: torch.Tensor, T: torch.Tensor,
                 lens: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> None:
    """A chunk's whole selection step (``ca_select_chunk``): pool the chunk's new
    key blocks into kbar and its Q-blocks into qbar, score, take the top-k
    mask and build the union tables T / lens, in four launches; every output
    buffer is the caller's (qbar [B, H_q, NQ, D], kbar [B, H_kv, NKB, D] kept
    across chunks, scores / mask [B, H_q, NQ, NKB], T [B, H_kv, NKB], lens [B, H_kv]).
    prior_len / chunk_len as device int32 [B] tensors use ``ca_select_chunk_devlen``
    (the kernels read them when they run)."""
    _need_cuda("q_chunk", q_chunk)
    if q_chunk.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q_chunk must be bfloat16 or float32")
    _need_cuda("k_cache", k_cache, q_chunk.dtype)
    for name, t, dt in (("qbar", qbar, torch.float32), ("kbar", kbar, torch.float32),
                        ("scores", scores, torch.float32), ("mask", mask, torch.uint8),
                        ("T", T, torch.int32), ("lens", lens, torch.int32)):
        _need_cuda(name, t, dt)
    if q_chunk.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q_chunk must be [B, H_q, C_max, D] and k_cache [B, H_kv, L, D]")
    B, H_q, C_max, D = q_chunk.shape
    H_kv, L = k_cache.shape[1], k_cache.shape[2]
    NQ, NKB = qbar.shape[2], kbar.shape[2]
    if tuple(qbar.shape) != (B, H_q, NQ, D) or tuple(kbar.shape) != (B, H_kv, NKB, D) or \
            tuple(scores.shape) != (B, H_q, NQ, NKB) or tuple(mask.shape) != (B, H_q, NQ, NKB) or \
            tuple(T.shape) != (B, H_kv, NKB) or tuple(lens.shape) != (B, H_kv):
        raise ValueError("qbar / kbar / scores / mask / T / lens shapes do not match")
    dt = _lib.CA_BF16 if q_chunk.dtype == torch.bfloat16 else _lib.CA_F32
    fn, pr, ch = _select_lengths("ca_select_chunk", prior_len, chunk_len, B)
    st = getattr(_lib.lib(), fn)(
        q_chunk.data_ptr(), k_cache.data_ptr(), dt, B, H_q, H_kv, C_max, L, D, pr, ch,
        int(budget), int(local), qbar.data_ptr(), NQ, kbar.data_ptr(), NKB, scores.data_ptr(),
        mask.data_ptr(), T.data_ptr(), lens.data_ptr(), _stream_ptr(stream))
    _lib.check(st, fn)


def append_select_chunk(k_new: torch.Tensor, v_new: torch.Tensor, q_chunk: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor, prior_len: Sequence[int],
                        chunk_len: Sequence[int], budget: int, local: int, qbar: torch.Tensor,
                        kbar: torch.Tensor, scores: torch.Tensor, mask: torch.Tensor,
                        T: torch.Tensor, lens: torch.Tensor,
                        stream: Optional[torch.cuda.Stream] = None) -> None:
    """``append_kv`` then ``select_chunk`` in the selection's four launches
    (``ca_append_select_chunk``): the first launch also writes the chunk's keys
    and values (k_new, v_new [B, H_kv, C_max, D]) into the caches and pools the
    new key blocks from them.  Same outputs as the two calls, bit for bit.
    prior_len / chunk_len as device int32 [B] tensors use
    ``ca_append_select_chunk_devlen``."""
    _need_cuda("k_new", k_new)
    if k_new.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("k_new must be bfloat16 or float32")
    for name, t in (("v_new", v_new), ("q_chunk", q_chunk), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        _need_cuda(name, t, k_new.dtype)
    for name, t, dt in (("qbar", qbar, torch.float32), ("kbar", kbar, torch.float32),
                        ("scores", scores, torch.float32), ("mask", mask, torch.uint8),
                        ("T", T, torch.int32), ("lens", lens, torch.int32)):
        _need_cuda(name, t, dt)
    if q_chunk.dim() != 4 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q_chunk must be [B, H_q, C_max, D] and the caches [B, H_kv, L, D]")
    B, H_q, C_max, D = q_chunk.shape
    H_kv, L = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_new.shape) != (B, H_kv, C_max, D) or v_new.shape != k_new.shape or \
            k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("k_new / v_new must be [B, H_kv, C_max, D] of the caches and q_chunk")
    NQ, NKB = qbar.shape[2], kbar.shape[2]
    if tuple(qbar.shape) != (B, H_q, NQ, D) or tuple(kbar.shape) != (B, H_kv, NKB, D) or \
            tuple(scores.shape) != (B, H_q, NQ, NKB) or tuple(mask.shape) != (B, H_q, NQ, NKB) or \
            tuple(T.shape) != (B, H_kv, NKB) or tuple(lens.shape) != (B, H_kv):
        raise ValueError("qbar / kbar / scores / mask / T / lens shapes do not match")
    dt = _lib.CA_BF16 if q_chunk.dtype == torch.bfloat16 else _lib.CA_F32
    fn, pr, ch = _select_lengths("ca_append_select_chunk", prior_len, chunk_len, B)
    st = getattr(_lib.lib(), fn)(
        k_new.data_ptr(), v_new.data_ptr(), q_chunk.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), dt, B, H_q, H_kv, C_max, L, D, pr, ch,
        int(budget), int(local), qbar.data_ptr(), NQ, kbar.data_ptr(), NKB, scores.data_ptr(),
        mask.data_ptr(), T.data_ptr(), lens.data_ptr(), _stream_ptr(stream))
    _lib.check(st, fn)
