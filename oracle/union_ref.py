"""Block-Union KV selection, written as its set definition.

CompactAttention, "Methodology" / selection stage (technical summaries) and
the abstract: a per-head 2D (Q-block x KV-block) mask is reduced first over
the Q-blocks of the current chunk (one KV list serves a group of Q-blocks that
execute together) and then over the query heads that share one KV head (the
GQA group).  The result T[b,g] keeps every KV block that any Q-block or head
of the group selected (coverage) and nothing else (the minimal table), so

    T[b,g] = { kb < n_kv_blocks[b] :
               exists h in group g, qb < n_q_blocks[b] with mask[b,h,qb,kb] != 0 }.

Readings where the pages are silent: query head h belongs to group h // G with
G = H_q / H_kv (consecutive heads share a KV head); T is stored strictly
ascending and padded with -1 to NKB_max; cells outside a sequence's extent
(qb >= n_q_blocks[b] or kb >= n_kv_blocks[b]) are ignored; any nonzero byte
counts as selected.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def union_tables_ref(mask: np.ndarray, H_kv: int, n_q_blocks: Sequence[int],
                     n_kv_blocks: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """mask uint8 [B, H_q, NQ_max, NKB_max] -> (T int32 [B, H_kv, NKB_max], len int32 [B, H_kv])."""
    mask = np.asarray(mask)
    B, H_q, NQ_max, NKB_max = mask.shape
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    T = np.full((B, H_kv, NKB_max), -1, np.int32)
    ln = np.zeros((B, H_kv), np.int32)
    for b in range(B):
        nq = int(n_q_blocks[b])
        nkb = int(n_kv_blocks[b])
        for g in range(H_kv):
            cells = mask[b, g * G:(g + 1) * G, :nq, :nkb] != 0
            # any() over axis 1 is the Q-block union, over axis 0 the intra-group union
            selected = cells.any(axis=(0, 1))
            blocks = np.flatnonzero(selected)
            T[b, g, :blocks.size] = blocks
            ln[b, g] = blocks.size
    return T, ln


def tables_to_csr_ref(T: np.ndarray, ln: np.ndarray, L: int, block: int = 64):
    """Paged-metadata view of the tables (execution stage: the tables travel as
    kv_indptr / kv_indices to a paged dense kernel).  Pseudo-request u = b*H_kv+g;
    kv_indptr[u] = sum of len over earlier pseudo-requests; kv_indices holds the
    global page id u*(L/block) + T[b,g,j] of the cache viewed as
    [B*H_kv*L/block, block, D]."""
    B, H_kv, _ = T.shape
    flat_len = ln.reshape(-1).astype(np.int64)
    indptr = np.zeros(B * H_kv + 1, np.int32)
    indptr[1:] = np.cumsum(flat_len)
    pages = L // block
    parts = []
    for u in range(B * H_kv):
        b, g = divmod(u, H_kv)
        parts.append(u * pages + T[b, g, :ln[b, g]].astype(np.int64))
    indices = np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)
    return indptr, indices


def check_tables_ref(T: np.ndarray, ln: np.ndarray, n_kv_blocks, NKB_max: int) -> np.ndarray:
    """The table contract that attention relies on (selection-stage output,
    "Methodology": one minimal table per group, here read as strictly ascending
    block ids padded with -1), checked row by row in plain Python.  Returns
    int32 [B, H_kv]: 0 for a well-formed row, else the OR of 1 (len outside
    [0, NKB_max]), 2 (an entry j < len outside [0, n_kv_blocks[b])), 4 (the
    first len entries not strictly ascending), 8 (an entry past len other than
    -1); entries are judged against len clamped to [0, NKB_max]."""
    B, H_kv, _ = T.shape
    out = np.zeros((B, H_kv), np.int32)
    for b in range(B):
        for g in range(H_kv):
            n = int(ln[b, g])
            f = 0 if 0 <= n <= NKB_max else 1
            n = min(max(n, 0), NKB_max)
            row = [int(x) for x in T[b, g]]
            for j in range(NKB_max):
                if j < n:
                    if not 0 <= row[j] < int(n_kv_blocks[b]):
                        f |= 2
                    if j > 0 and row[j] <= row[j - 1]:
                        f |= 4
                elif row[j] != -1:
                    f |= 8
            out[b, g] = f
    return out
