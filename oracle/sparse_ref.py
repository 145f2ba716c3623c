"""Block-sparse-kernel execution of the mask, written as its definition.

CompactAttention, abstract and "Methodology": existing block-sparse methods
hand the 2D (Q-block x KV-block) mask to a sparse kernel as its execution
plan, so each Q-block of each head attends exactly the KV blocks of its own
mask row; the union instead reads the mask as selection signals and widens
every row of a group to the group's table.  The baseline therefore computes,
for query head h of sequence b and chunk row i (Q-block qb = i // 64,
absolute position p = prior[b] + i),

    A_sparse(b,h,i) = { t : mask[b,h,qb,t//64] != 0,  t <= p,  t < prior[b] + chunk[b] }

and ordinary softmax attention over it, with the same conventions as the
union attention (scale applied to Q.K, natural-log LSE, empty set or padding
row -> O = 0 and LSE = -inf).  Float64 inside, float32 out.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .attention_ref import BLOCK, _as64, _softmax_attend, admissible_keys


def _row_blocks(mask_row: np.ndarray, nkb: int):
    blocks = np.flatnonzero(np.asarray(mask_row[:nkb]) != 0).astype(np.int32)
    return blocks, blocks.size


def sparse_attention_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                         prior: Sequence[int], chunk: Sequence[int], scale: float
                         ) -> Tuple[np.ndarray, np.ndarray]:
    """q [B,H_q,C_max,D]; k, v [B,H_kv,L,D]; mask uint8 [B,H_q,NQ_max,NKB_max].
    Returns O float32 [B,H_q,C_max,D] and lse float32 [B,H_q,C_max]."""
    B, H_q, C_max, D = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    O = np.zeros((B, H_q, C_max, D), np.float32)
    lse = np.full((B, H_q, C_max), -np.inf, np.float32)
    for b in range(B):
        P, C = int(prior[b]), int(chunk[b])
        nkb = -(-(P + C) // BLOCK)
        for h in range(H_q):
            g = h // G
            for qb in range(-(-C // BLOCK)):
                blocks, n = _row_blocks(mask[b, h, qb], nkb)
                keys = admissible_keys(blocks, n, P, C, P + C - 1)
                rows = np.arange(qb * BLOCK, min((qb + 1) * BLOCK, C))
                o, l_ = _softmax_attend(_as64(q[b, h, rows]), _as64(k[b, g, keys]),
                                        _as64(v[b, g, keys]), keys, P + rows, scale)
                O[b, h, rows] = o
                lse[b, h, rows] = l_
    return O, lse


def sparse_attention_rows_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                              prior: Sequence[int], chunk: Sequence[int], scale: float,
                              rows: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """The same definition at sampled outputs ``rows`` (int [n,3] of (b, h, i))."""
    rows = np.asarray(rows, np.int64).reshape(-1, 3)
    H_q, D = q.shape[1], q.shape[3]
    G = H_q // k.shape[1]
    O = np.zeros((rows.shape[0], D), np.float32)
    lse = np.full(rows.shape[0], -np.inf, np.float32)
    groups = {}
    for n, (b, h, i) in enumerate(rows):
        groups.setdefault((int(b), int(h), int(i) // BLOCK), []).append(n)
    for (b, h, qb), idx in groups.items():
        P, C = int(prior[b]), int(chunk[b])
        idx = np.asarray(idx)
        live = idx[rows[idx, 2] < C]
        if not live.size:
            continue
        blocks, n = _row_blocks(mask[b, h, qb], -(-(P + C) // BLOCK))
        keys = admissible_keys(blocks, n, P, C, P + C - 1)
        g = h // G
        o, l_ = _softmax_attend(_as64(q[b, h, rows[live, 2]]), _as64(k[b, g, keys]),
                                _as64(v[b, g, keys]), keys, P + rows[live, 2], scale)
        O[live] = o
        lse[live] = l_
    return O, lse
