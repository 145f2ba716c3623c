"""Explicit KV compaction, written as its definition.

CompactAttention, abstract: the per-group block tables let the attention read
the selected KV blocks in place, with no explicit KV compaction; the KV copy
that token-level selection pays is the overhead this avoids.  The baseline
measured against zero-copy execution is that copy: for each (b, g), the
selected blocks of the accumulated (prior) cache are gathered into contiguous
blocks that end where the chunk starts, and the chunk's own blocks stay where
they are, so every key keeps its causal relation to every query:

    p       = #{ j < len[b,g] : T[b,g,j] < prior[b]/64 }
    dst(j)  = prior[b]/64 - p + j    for j < p     (prior blocks, packed)
    dst(j)  = T[b,g,j]               for j >= p    (chunk blocks, in place)
    K_out[b,g,dst(j)] = K[b,g,T[b,g,j]],  V likewise,  T_out[b,g,j] = dst(j).

Reading where the pages are silent: the gathered buffer keeps the cache's
[B, H_kv, L, D] layout (a dense kernel then runs on the contiguous table), and
the destination of each prior block is the one that keeps it before the chunk.
T is ascending (as the union produces it), so prior entries come first.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

BLOCK = 64


def compact_kv_ref(k: np.ndarray, v: np.ndarray, T: np.ndarray, ln: np.ndarray,
                   prior: Sequence[int], chunk: Sequence[int]
                   ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """k, v [B,H_kv,L,D]; T [B,H_kv,NKB_max] ascending; ln [B,H_kv].

    Returns (k_out, v_out, T_out, written): k_out/v_out hold zeros where no
    block was copied, ``written`` [B,H_kv,L/64] bool marks the copied blocks."""
    B, H_kv, L, D = k.shape
    NKB_max = T.shape[2]
    k_out = np.zeros_like(k)
    v_out = np.zeros_like(v)
    T_out = np.full((B, H_kv, NKB_max), -1, np.int32)
    written = np.zeros((B, H_kv, L // BLOCK), bool)
    for b in range(B):
        P_blk = int(prior[b]) // BLOCK
        nkb = (int(prior[b]) + int(chunk[b]) + BLOCK - 1) // BLOCK
        for g in range(H_kv):
            sel = [int(x) for x in T[b, g, :int(ln[b, g])]]
            p = sum(1 for kb in sel if 0 <= kb < P_blk)
            for j, kb in enumerate(sel):
                if not 0 <= kb < nkb:
                    continue
                dst = P_blk - p + j if kb < P_blk else kb
                if not 0 <= dst < nkb:
                    continue
                k_out[b, g, dst * BLOCK:(dst + 1) * BLOCK] = k[b, g, kb * BLOCK:(kb + 1) * BLOCK]
                v_out[b, g, dst * BLOCK:(dst + 1) * BLOCK] = v[b, g, kb * BLOCK:(kb + 1) * BLOCK]
                T_out[b, g, j] = dst
                written[b, g, dst] = True
    return k_out, v_out, T_out, written
