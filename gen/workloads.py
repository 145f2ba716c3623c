"""Synthetic workloads for one chunked-prefill attention call.

Every workload is one chunk of queries per sequence attending to a KV cache in
the KV-head-major layout ``[B, H_kv, L, D]`` (CompactAttention, execution
stage: each (batch, KV head, block) triple is one contiguous region), plus a
per-head 2D block mask ``[B, H_q, NQ_max, NKB_max]`` of 0/1 bytes (selection
stage: the mask a lightweight pattern search would hand over).

Shapes follow LLaMA-3.1-8B attention (32 query heads, 8 KV heads, head dim
128), the model the pages attach their 128K chunked-prefill speedup to
(CompactAttention abstract; "Experimental results" of the technical
summaries).  The pages print no block size; 64 tokens is used for both the
Q-block and the KV block.

Recipe (fixed so every consumer sees the same bytes):

* Two ``numpy.random.Generator(PCG64(...))`` streams: ``PCG64([seed, 0])``
  draws Q, then K, then V; ``PCG64([seed, 1])`` draws the mask, so a mask can
  be regenerated without drawing the tensors.
* Q, K, V ~ N(0, 1) drawn in float32; bf16 workloads round with torch's
  ``.to(torch.bfloat16)`` (round to nearest even).
* Q is drawn for all ``C_max`` rows.  K and V are drawn per sequence only for
  the rows ``[0, prior_b + chunk_b)`` that exist; the rest of the cache
  capacity is zero (tests may poison it).
* The current chunk's own K/V rows are already in the cache at
  ``[prior_b, prior_b + chunk_b)`` (chunked prefill appends before attending).
* Mask: prior-block cells are drawn per workload (below); the chunk's own
  blocks get the causal block triangle ``mask[qb, P_blk + j] = 1`` for
  ``j <= qb``, so every current-chunk block reaches the union and token-level
  causality is left to attention.  Cells outside a sequence's extent are 0.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np
import torch

BLOCK = 64  # tokens per KV block and per Q-block

VSLASH_DENSITIES = (0.02, 0.05, 0.1, 0.25, 0.5, 1.0)
VSLASH_HEAD_MODES = ("identical", "independent")


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str  # "f32" or "bf16"
    B: int
    H_q: int
    H_kv: int
    D: int
    prior: List[int]
    chunk: List[int]
    C_max: int
    L: int
    NQ_max: int
    NKB_max: int
    scale: float
    mask: np.ndarray  # uint8 [B, H_q, NQ_max, NKB_max]
    q: Optional[torch.Tensor] = None  # CPU [B, H_q, C_max, D]
    k: Optional[torch.Tensor] = None  # CPU [B, H_kv, L, D]
    v: Optional[torch.Tensor] = None
    meta: Dict[str, object] = dataclasses.field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def block(self) -> int:
        return BLOCK

    @property
    def n_q_blocks(self) -> List[int]:
        return [-(-c // BLOCK) for c in self.chunk]

    @property
    def n_kv_blocks(self) -> List[int]:
        return [-(-(p + c) // BLOCK) for p, c in zip(self.prior, self.chunk)]

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bit patterns (uint16/int16) to float32."""
    return (bits.astype(np.uint16).astype(np.uint32) << 16).view(np.float32)


def tensor_to_f32(t: torch.Tensor) -> np.ndarray:
    """CPU tensor (float32 or bfloat16) -> float32 ndarray holding the same values."""
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.contiguous().numpy()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.contiguous().view(torch.int16).numpy())
    raise TypeError(f"unsupported dtype {t.dtype}")


# --------------------------------------------------------------------------- masks


def _causal_triangle(mask_b: np.ndarray, prior: int, chunk: int) -> None:
    """mask_b [H_q, NQ_max, NKB_max]: mark, for each Q-block, the chunk's own KV
    blocks from the chunk start up to the block holding that Q-block's last row
    (for aligned chunks: the block triangle on and below the diagonal)."""
    p_blk = prior // BLOCK
    for qb in range(-(-chunk // BLOCK)):
        last = prior + min(BLOCK * qb + BLOCK - 1, chunk - 1)
        mask_b[:, qb, p_blk:last // BLOCK + 1] = 1


def _bernoulli_sink_local(rng, H_q, nq, p_blk, p, local, colshared=False, group=0):
    """Prior-block cells: Bernoulli(p) per (head, Q-block, KV-block) cell
    (``colshared``: one draw per (head, KV-block), same for every Q-block;
    ``group`` = G > 0: one draw per (group of G heads, KV-block), same for the
    group's heads and every Q-block), with block 0 (sink) and the last
    ``local`` prior blocks forced on."""
    if group:
        cells = rng.random((H_q // group, 1, 1, p_blk)) < p
        cells = np.broadcast_to(cells, (H_q // group, group, nq, p_blk)).reshape(H_q, nq, p_blk).copy()
    elif colshared:
        cells = rng.random((H_q, 1, p_blk)) < p
        cells = np.broadcast_to(cells, (H_q, nq, p_blk)).copy()
    else:
        cells = rng.random((H_q, nq, p_blk)) < p
    cells[:, :, 0] = True
    if local:
        cells[:, :, max(p_blk - local, 0):p_blk] = True
    return cells.astype(np.uint8)


def _vertical_slash_head(rng, nq, p_blk, d) -> np.ndarray:
    """One head's prior-block cells [nq, p_blk] for a vertical-slash pattern of
    nominal density d: n = round(d*p_blk) lines, ceil(n/2) vertical columns
    (block 0 plus distinct uniform columns in [1, p_blk)) and the rest slash
    lines at distinct offsets o in [nq, p_blk]; slash o marks (qb, p_blk+qb-o)."""
    cells = np.zeros((nq, p_blk), np.uint8)
    if d >= 1.0:
        cells[:] = 1
        return cells
    n = int(round(d * p_blk))
    n_v = -(-n // 2)
    n_s = n - n_v
    cols = [0]
    if n_v > 1:
        cols += list(rng.choice(np.arange(1, p_blk), n_v - 1, replace=False))
    cells[:, np.asarray(cols, np.int64)] = 1
    if n_s > 0:
        offs = rng.choice(np.arange(nq, p_blk + 1), n_s, replace=False)
        qb = np.arange(nq)
        for o in offs:
            cells[qb, p_blk + qb - int(o)] = 1
    return cells


# --------------------------------------------------------------------------- tensors


def _draw_qkv(rng, B, H_q, H_kv, D, prior, chunk, C_max, L, dtype):
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = torch.from_numpy(rng.standard_normal((B, H_q, C_max, D), dtype=np.float32)).to(tdt)
    caches = []
    for _ in range(2):  # K then V
        c = torch.zeros((B, H_kv, L, D), dtype=tdt)
        for b in range(B):
            n = prior[b] + chunk[b]
            if n:
                c[b, :, :n] = torch.from_numpy(
                    rng.standard_normal((H_kv, n, D), dtype=np.float32)).to(tdt)
        caches.append(c)
    return q, caches[0], caches[1]


def _round_up(x, m):
    return -(-x // m) * m


def make_custom(B: int, H_q: int, H_kv: int, D: int, prior: Sequence[int],
                chunk: Sequence[int], dtype: str, seed: int,
                cell_fn: Callable, C_max: Optional[int] = None, L: Optional[int] = None,
                NKB_max: Optional[int] = None, name: str = "custom",
                with_tensors: bool = True, triangle: bool = True,
                tensor_seed: Optional[int] = None) -> Workload:
    """General workload.  ``cell_fn(rng, b, H_q, nq, p_blk) -> uint8 [H_q, nq, p_blk]``
    gives the prior-block cells of sequence b.  Q/K/V come from ``tensor_seed``
    (default: ``seed``), the mask from ``seed``."""
    prior = [int(p) for p in prior]
    chunk = [int(c) for c in chunk]
    C_max = int(C_max if C_max is not None else max(chunk))
    tot = [p + c for p, c in zip(prior, chunk)]
    L = int(L if L is not None else _round_up(max(tot), BLOCK))
    nq_max = -(-C_max // BLOCK)
    nkb = [-(-t // BLOCK) for t in tot]
    NKB_max = int(NKB_max if NKB_max is not None else max(nkb))
    if with_tensors:
        ts = seed if tensor_seed is None else tensor_seed
        rng_t = np.random.Generator(np.random.PCG64([ts, 0]))
        q, k, v = _draw_qkv(rng_t, B, H_q, H_kv, D, prior, chunk, C_max, L, dtype)
    else:
        q = k = v = None
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    mask = np.zeros((B, H_q, nq_max, NKB_max), np.uint8)
    for b in range(B):
        nq = -(-chunk[b] // BLOCK)
        p_blk = prior[b] // BLOCK
        if p_blk:
            mask[b, :, :nq, :p_blk] = cell_fn(rng, b, H_q, nq, p_blk)
        if triangle:
            _causal_triangle(mask[b], prior[b], chunk[b])
    return Workload(name=name, dtype=dtype, B=B, H_q=H_q, H_kv=H_kv, D=D, prior=prior,
                    chunk=chunk, C_max=C_max, L=L, NQ_max=nq_max, NKB_max=NKB_max,
                    scale=1.0 / math.sqrt(D), mask=mask, q=q, k=k, v=v)


# --------------------------------------------------------------------------- named workloads

WORKLOADS = ("tiny_f32", "llama8b_32k", "llama8b_128k", "ragged_b4", "vslash_128k")


def make_workload(name: str, variant: Optional[str] = None, density: Optional[float] = None,
                  heads: str = "independent", seed: Optional[int] = None,
                  with_tensors: bool = True) -> Workload:
    """Named workloads.

    tiny_f32      fp32, B=1, 4 query heads / 1 KV head, D=64; 1024 prior tokens +
                  a 256-token chunk; prior cells Bernoulli(0.25), block 0 forced.
    llama8b_32k   bf16, B=1, 32/8 heads, D=128; 30720 prior + 2048-token chunk;
                  sink + last 4 prior blocks + Bernoulli(0.15).
    llama8b_128k  bf16, as above with 129024 prior tokens; sink + last 8 prior
                  blocks + Bernoulli(0.05) drawn per head.  variant "pairwise"
                  (default: one draw per (head, Q-block, KV-block) cell),
                  "colshared" (one draw per (head, KV-block), shared by all
                  Q-blocks), "groupshared" (one draw per (KV group, KV-block),
                  shared by the group's heads and all Q-blocks: every mask row
                  of a group equals the group's union), or "dense" (all-ones
                  mask: the dense baseline).
    ragged_b4     bf16, B=4, prior {16384, 32768, 65536, 126976} + 1024-token
                  chunk each, cache capacity 128000; per-sequence density
                  p_b ~ U[0.05, 0.3]; sink + last 4 prior blocks forced.
    vslash_128k   bf16, 128K shape (Q/K/V of llama8b_128k); vertical-slash mask
                  of nominal density ``density`` with the heads of a group
                  ``identical`` or ``independent`` (mask seed
                  5000 + 10 * density index + head mode).
    """
    if name == "tiny_f32":
        s = 1001 if seed is None else seed
        w = make_custom(1, 4, 1, 64, [1024], [256], "f32", s,
                        lambda rng, b, H, nq, pb: _bernoulli_sink_local(rng, H, nq, pb, 0.25, 0),
                        name=name, with_tensors=with_tensors)
        w.meta.update(mask="bernoulli", p=0.25)
        return w
    if name == "llama8b_32k":
        s = 1002 if seed is None else seed
        w = make_custom(1, 32, 8, 128, [30720], [2048], "bf16", s,
                        lambda rng, b, H, nq, pb: _bernoulli_sink_local(rng, H, nq, pb, 0.15, 4),
                        name=name, with_tensors=with_tensors)
        w.meta.update(mask="bernoulli", p=0.15, local=4)
        return w
    if name == "llama8b_128k":
        s = 1003 if seed is None else seed
        variant = variant or "pairwise"
        if variant == "dense":
            fn = lambda rng, b, H, nq, pb: np.ones((H, nq, pb), np.uint8)  # noqa: E731
        elif variant in ("pairwise", "colshared", "groupshared"):
            cs = variant == "colshared"
            grp = 4 if variant == "groupshared" else 0
            fn = lambda rng, b, H, nq, pb: _bernoulli_sink_local(  # noqa: E731
                rng, H, nq, pb, 0.05, 8, colshared=cs, group=grp)
        else:
            raise ValueError(f"unknown variant {variant}")
        w = make_custom(1, 32, 8, 128, [129024], [2048], "bf16", s, fn, name=name,
                        with_tensors=with_tensors)
        if variant == "dense":
            w.mask[:] = 1
        w.meta.update(mask=variant, p=0.05, local=8)
        return w
    if name == "ragged_b4":
        s = 1004 if seed is None else seed
        prior = [16384, 32768, 65536, 126976]
        dens: List[float] = []

        def fn(rng, b, H, nq, pb):
            if b == 0:
                dens.extend(float(x) for x in rng.uniform(0.05, 0.3, size=4))
            return _bernoulli_sink_local(rng, H, nq, pb, dens[b], 4)

        w = make_custom(4, 32, 8, 128, prior, [1024] * 4, "bf16", s, fn, L=128000,
                        name=name, with_tensors=with_tensors)
        w.meta.update(mask="bernoulli", p=dens, local=4)
        return w
    if name == "vslash_128k":
        if density is None:
            density = 0.1
        di = VSLASH_DENSITIES.index(density)
        hm = VSLASH_HEAD_MODES.index(heads)
        s = 1000 * 5 + 10 * di + hm if seed is None else seed
        G = 4

        def fn(rng, b, H, nq, pb):
            out = np.zeros((H, nq, pb), np.uint8)
            if heads == "identical":
                for g in range(H // G):
                    out[g * G:(g + 1) * G] = _vertical_slash_head(rng, nq, pb, density)[None]
            else:
                for h in range(H):
                    out[h] = _vertical_slash_head(rng, nq, pb, density)
            return out

        # Q/K/V are those of llama8b_128k (seed 1003); only the mask varies per sweep point
        w = make_custom(1, 32, 8, 128, [129024], [2048], "bf16", s, fn, name=name,
                        with_tensors=with_tensors, tensor_seed=1003)
        if density >= 1.0:
            w.mask[:] = 1
        w.meta.update(mask="vertical_slash", density=density, heads=heads)
        return w
    raise ValueError(f"unknown workload {name}")
