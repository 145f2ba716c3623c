"""A lightweight block-mask producer, written as its definition.

CompactAttention, "Methodology" (selection stage) and the problem statement
of the technical summaries: the union consumes a per-head 2D block mask made
by whatever cheap searcher the caller uses, and that search is repeated over the
growing KV cache at every chunk.  The pages leave the searcher open (they name
trained and training-free ones from other work).  The stand-in here is a
training-free one whose result has a plain definition:

  pooled query  qbar[b,h,qb] = mean of the 64 rows of Q-block qb of head h
  pooled key    kbar[b,g,kb] = mean of the 64 rows of KV block kb of KV head g
  block score   s[b,h,qb,kb] = qbar[b,h,qb] . kbar[b,g,kb]     (g = h // G)

  mask[b,h,qb,kb] = 1  for the sink block kb = 0, the last `local` prior
                       blocks, the chunk's causal block triangle
                       (kb = P/64 + j, j <= qb), and the `budget` highest-
                       scoring remaining prior blocks (ties: lower kb first);
                  = 0  elsewhere, and on every Q-block qb >= chunk/64.

Readings: the softmax scale does not change the ranking and is left out; the
candidates are the prior blocks 1 .. P/64 - local - 1; with fewer candidates
than the budget, all are taken.  Pooling and scores are float64 here; the
selection step is a separate function so that a test can give it any scores.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

BLOCK = 64


def pool_blocks_ref(x: np.ndarray, blk_begin: Sequence[int], blk_end: Sequence[int],
                    n_out: int) -> np.ndarray:
    """x [B,H,R,D] -> float64 [B,H,n_out,D]: entry kb is the mean of rows
    64kb .. 64kb+63 for blk_begin[b] <= kb < blk_end[b], NaN elsewhere."""
    B, H, R, D = x.shape
    out = np.full((B, H, n_out, D), np.nan)
    for b in range(B):
        for kb in range(int(blk_begin[b]), int(blk_end[b])):
            out[b, :, kb] = np.asarray(x[b, :, kb * BLOCK:(kb + 1) * BLOCK], np.float64).mean(axis=1)
    return out


def block_scores_ref(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """qbar [B,H_q,NQ,D], kbar [B,H_kv,NKB,D] -> s [B,H_q,NQ,NKB] = qbar . kbar."""
    B, H_q, NQ, D = qbar.shape
    H_kv = kbar.shape[1]
    G = H_q // H_kv
    s = np.zeros((B, H_q, NQ, kbar.shape[2]))
    for b in range(B):
        for h in range(H_q):
            s[b, h] = np.asarray(qbar[b, h], np.float64) @ np.asarray(kbar[b, h // G], np.float64).T
    return s


def topk_mask_ref(scores: np.ndarray, prior: Sequence[int], chunk: Sequence[int], budget: int,
                  local: int, NKB_max: int) -> np.ndarray:
    """Selection from given scores [B,H_q,NQ_max,>=P/64] -> uint8 mask
    [B,H_q,NQ_max,NKB_max] (definition in the module docstring)."""
    B, H_q, NQ_max = scores.shape[:3]
    mask = np.zeros((B, H_q, NQ_max, NKB_max), np.uint8)
    for b in range(B):
        pblk, nq = int(prior[b]) // BLOCK, int(chunk[b]) // BLOCK
        lo_local = max(pblk - local, 1)
        cand = np.arange(1, lo_local)
        for h in range(H_q):
            for qb in range(nq):
                row = mask[b, h, qb]
                if pblk:
                    row[0] = 1
                    row[lo_local:pblk] = 1
                if cand.size:
                    s = scores[b, h, qb, cand]
                    order = sorted(range(cand.size), key=lambda i: (-s[i], cand[i]))
                    row[cand[order[:budget]]] = 1
                row[pblk:pblk + qb + 1] = 1
    return mask


def producer_mask_ref(q: np.ndarray, k: np.ndarray, prior: Sequence[int], chunk: Sequence[int],
                      budget: int, local: int, NKB_max: int) -> np.ndarray:
    """The whole producer: q [B,H_q,C_max,D], k [B,H_kv,L,D] -> uint8 mask."""
    B = q.shape[0]
    NQ_max = -(-q.shape[2] // BLOCK)
    qbar = pool_blocks_ref(q, [0] * B, [int(c) // BLOCK for c in chunk], NQ_max)
    n_kb = max(int(p) // BLOCK for p in prior) or 1
    kbar = pool_blocks_ref(k, [0] * B, [int(p) // BLOCK for p in prior], n_kb)
    s = block_scores_ref(np.nan_to_num(qbar), np.nan_to_num(kbar))
    return topk_mask_ref(s, prior, chunk, budget, local, NKB_max)
