"""Chunk attention over the union blocks, written as its definition.

CompactAttention, execution stage (technical summaries, "Methodology"): the
per-group tables are handed to a paged *dense* attention kernel that reads the
selected KV blocks in place from a KV-head-major [B, H_kv, L, D] cache.  What
that computes, for query head h (group g = h // G) of sequence b and chunk row
i at absolute position p = prior[b] + i, is ordinary softmax attention over

    A(b,h,i) = { t : floor(t/64) in T[b,g],  t <= p,  t < prior[b] + chunk[b] }

(chunked prefill: the chunk's queries see the accumulated cache and, causally,
their own chunk, whose K/V were appended before attending).

    x_t  = scale * sum_d Q[b,h,i,d] * K[b,g,t,d]
    O    = sum_{t in A} softmax(x)_t * V[b,g,t,:]      (max-subtracted)
    LSE  = log sum_{t in A} exp(x_t)                    (natural log)

Readings where the pages are silent: scale = 1/sqrt(D); an empty A gives
O = 0 and LSE = -inf; chunk rows i >= chunk[b] (padding up to C_max) give
O = 0 and LSE = -inf.  All arithmetic is float64; outputs are float32.
The oracle may gather the selected keys into a temporary array: only the GPU
path must read them in place.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

BLOCK = 64


def admissible_keys(T_bg: np.ndarray, len_bg: int, prior_b: int, chunk_b: int,
                    pos_max: int) -> np.ndarray:
    """All keys t of the blocks listed in T_bg[:len_bg] with t < prior+chunk and
    t <= pos_max, in ascending block order (ascending t when T_bg is ascending)."""
    blocks = np.asarray(T_bg[:len_bg], np.int64)
    keys = (blocks[:, None] * BLOCK + np.arange(BLOCK, dtype=np.int64)[None, :]).reshape(-1)
    keep = (keys < prior_b + chunk_b) & (keys <= pos_max)
    return keys[keep]


def _softmax_attend(q_rows: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray,
                    keys: np.ndarray, pos: np.ndarray, scale: float):
    """q_rows [n,D], k_sel/v_sel [m,D] (rows of the keys in ``keys``), pos [n]
    absolute query positions.  Returns (O [n,D], lse [n]) in float64."""
    n = q_rows.shape[0]
    D = v_sel.shape[1] if v_sel.ndim == 2 else q_rows.shape[1]
    if keys.size == 0:
        return np.zeros((n, D)), np.full(n, -np.inf)
    x = scale * (q_rows @ k_sel.T)
    ok = keys[None, :] <= pos[:, None]
    x = np.where(ok, x, -np.inf)
    has = ok.any(axis=1)
    m = np.where(has, x.max(axis=1), 0.0)
    e = np.exp(x - m[:, None])  # masked entries: exp(-inf) = 0
    s = e.sum(axis=1)
    s_safe = np.where(has, s, 1.0)
    out = (e @ v_sel) / s_safe[:, None]
    out[~has] = 0.0
    lse = np.where(has, m + np.log(s_safe), -np.inf)
    return out, lse


def _as64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def chunk_attention_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, T: np.ndarray,
                        ln: np.ndarray, prior: Sequence[int], chunk: Sequence[int],
                        scale: float, slab: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """Full chunk attention.  q [B,H_q,C_max,D]; k, v [B,H_kv,L,D]; T/ln from the
    union.  Returns O float32 [B,H_q,C_max,D] and lse float32 [B,H_q,C_max]."""
    B, H_q, C_max, D = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    O = np.zeros((B, H_q, C_max, D), np.float32)
    lse = np.full((B, H_q, C_max), -np.inf, np.float32)
    for b in range(B):
        P, C = int(prior[b]), int(chunk[b])
        for g in range(H_kv):
            keys = admissible_keys(T[b, g], int(ln[b, g]), P, C, P + C - 1)
            k_sel = _as64(k[b, g, keys])
            v_sel = _as64(v[b, g, keys])
            for h in range(g * G, (g + 1) * G):
                for i0 in range(0, C, slab):
                    rows = np.arange(i0, min(i0 + slab, C))
                    o, l_ = _softmax_attend(_as64(q[b, h, rows]), k_sel, v_sel, keys,
                                            P + rows, scale)
                    O[b, h, rows] = o
                    lse[b, h, rows] = l_
    return O, lse


def chunk_attention_rows_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, T: np.ndarray,
                             ln: np.ndarray, prior: Sequence[int], chunk: Sequence[int],
                             scale: float, rows: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """The same definition evaluated only at sampled outputs ``rows`` (int [n,3] of
    (b, h, i)).  Returns O [n,D] float32 and lse [n] float32."""
    rows = np.asarray(rows, np.int64).reshape(-1, 3)
    H_q, D = q.shape[1], q.shape[3]
    H_kv = k.shape[1]
    G = H_q // H_kv
    O = np.zeros((rows.shape[0], D), np.float32)
    lse = np.full(rows.shape[0], -np.inf, np.float32)
    by_bg = {}
    for n, (b, h, i) in enumerate(rows):
        by_bg.setdefault((int(b), int(h) // G), []).append(n)
    for (b, g), idx in by_bg.items():
        P, C = int(prior[b]), int(chunk[b])
        keys = admissible_keys(T[b, g], int(ln[b, g]), P, C, P + C - 1)
        k_sel = _as64(k[b, g, keys])
        v_sel = _as64(v[b, g, keys])
        idx = np.asarray(idx)
        live = idx[rows[idx, 2] < C]
        if live.size:
            qr = _as64(q[rows[live, 0], rows[live, 1], rows[live, 2]])
            o, l_ = _softmax_attend(qr, k_sel, v_sel, keys, P + rows[live, 2], scale)
            O[live] = o
            lse[live] = l_
    return O, lse


def chunk_attention_dense_masked_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                                     T: np.ndarray, ln: np.ndarray, prior: Sequence[int],
                                     chunk: Sequence[int], scale: float):
    """Second formulation of the same result: dense logits over every cached key
    t < prior+chunk, set to -inf where floor(t/64) is not in T[b,g] or t > p."""
    B, H_q, C_max, D = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    O = np.zeros((B, H_q, C_max, D), np.float32)
    lse = np.full((B, H_q, C_max), -np.inf, np.float32)
    for b in range(B):
        P, C = int(prior[b]), int(chunk[b])
        n_tok = P + C
        t = np.arange(n_tok)
        for h in range(H_q):
            g = h // G
            in_T = np.zeros(-(-n_tok // BLOCK) + 1, bool)
            sel = np.asarray(T[b, g, :ln[b, g]], np.int64)
            in_T[sel[sel < in_T.size]] = True
            if C == 0:
                continue
            x = scale * (_as64(q[b, h, :C]) @ _as64(k[b, g, :n_tok]).T)
            ok = in_T[t // BLOCK][None, :] & (t[None, :] <= (P + np.arange(C))[:, None])
            x = np.where(ok, x, -np.inf)
            has = ok.any(axis=1)
            m = np.where(has, x.max(axis=1), 0.0)
            e = np.exp(x - m[:, None])
            s = np.where(has, e.sum(axis=1), 1.0)
            o = (e @ _as64(v[b, g, :n_tok])) / s[:, None]
            o[~has] = 0.0
            O[b, h, :C] = o
            lse[b, h, :C] = np.where(has, m + np.log(s), -np.inf)
    return O, lse
