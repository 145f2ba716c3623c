"""Chunk-by-chunk driver of the whole path over a growing KV cache.

Chunked prefill (CompactAttention, problem statement and "Methodology" of the
technical summaries): a long prompt is processed in fixed-size chunks; for
each one the chunk's keys and values are already appended to the cache, a
lightweight search makes the per-head block mask over the cache so far, the
union turns it into per-group tables, and zero-copy attention runs the
chunk's queries over the selected blocks.  Every step is a call into the HIP
library; this class only keeps the per-prompt buffers (allocated once, reused
by every chunk) and issues the calls in order on one stream.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import (balanced_workspace_size, block_mask_topk, build_union_tables, chunk_attention,
               pool_blocks)
from ._lib import CA_BLOCK


class ChunkedPrefill:
    """Per-prompt state: caches [B, H_kv, L, D] (device, bf16 or fp32; the
    prompt's keys/values up to the current chunk must be in place), pooled
    keys kept across chunks, and the mask / table / output buffers.

    ``step(q_chunk, prior)`` runs one chunk of C tokens at absolute offset
    ``prior``; ``step_dense`` runs the same attention over every block (the
    dense baseline).  ``balanced`` runs the sparse attention through
    ``chunk_attention(..., balanced=True)``: the union's per-group tables differ
    in length from group to group, and the plan spreads that work evenly over
    the compute units (the workspace is allocated here, once)."""

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, H_q: int, C: int,
                 budget: int, local: int, scale: Optional[float] = None,
                 balanced: bool = False):
        B, H_kv, L, D = k_cache.shape
        if C % CA_BLOCK or L % CA_BLOCK:
            raise ValueError("chunk length and cache capacity must be multiples of 64")
        dev = k_cache.device
        self.k, self.v = k_cache, v_cache
        self.B, self.H_q, self.H_kv, self.L, self.D, self.C = B, H_q, H_kv, L, D, C
        self.budget, self.local = int(budget), int(local)
        self.scale = scale if scale is not None else 1.0 / math.sqrt(D)
        self.NQ = C // CA_BLOCK
        self.NKB = L // CA_BLOCK
        self.kbar = torch.zeros((B, H_kv, self.NKB, D), dtype=torch.float32, device=dev)
        self.qbar = torch.zeros((B, H_q, self.NQ, D), dtype=torch.float32, device=dev)
        self.scores = torch.empty((B, H_q, self.NQ, self.NKB), dtype=torch.float32, device=dev)
        self.mask = torch.empty((B, H_q, self.NQ, self.NKB), dtype=torch.uint8, device=dev)
        self.T = torch.empty((B, H_kv, self.NKB), dtype=torch.int32, device=dev)
        self.lens = torch.empty((B, H_kv), dtype=torch.int32, device=dev)
        self.T_dense = torch.arange(self.NKB, dtype=torch.int32, device=dev).repeat(B * H_kv, 1) \
            .view(B, H_kv, self.NKB)
        self.out = torch.empty((B, H_q, C, D), dtype=k_cache.dtype, device=dev)
        self.balanced = bool(balanced)
        self.ws = None
        if self.balanced:
            self.ws = torch.empty(balanced_workspace_size(B, H_q, H_kv, C, D), dtype=torch.uint8,
                                  device=dev)

    def select(self, q_chunk: torch.Tensor, prior: int, stream=None) -> None:
        """Pool the chunk's new key blocks and its queries, make the mask and
        build the union tables (into self.mask / self.T / self.lens)."""
        B, C = self.B, self.C
        p_blk, n_blk = prior // CA_BLOCK, (prior + C) // CA_BLOCK
        pool_blocks(self.k, [p_blk] * B, [n_blk] * B, out=self.kbar, stream=stream)
        pool_blocks(q_chunk, [0] * B, [self.NQ] * B, out=self.qbar, stream=stream)
        block_mask_topk(self.qbar, self.kbar, [prior] * B, [C] * B, self.budget, self.local,
                        scores=self.scores, mask=self.mask, stream=stream)
        build_union_tables(self.mask, self.H_kv, [self.NQ] * B, [n_blk] * B, T=self.T,
                           lens=self.lens, stream=stream)

    def attend(self, q_chunk: torch.Tensor, prior: int, out=None, stream=None) -> torch.Tensor:
        out = self.out if out is None else out
        return chunk_attention(q_chunk, self.k, self.v, self.T, self.lens, [prior] * self.B,
                               [self.C] * self.B, self.scale, out=out, stream=stream,
                               balanced=self.balanced, workspace=self.ws)

    def step(self, q_chunk: torch.Tensor, prior: int, out=None, stream=None) -> torch.Tensor:
        self.select(q_chunk, prior, stream)
        return self.attend(q_chunk, prior, out, stream)

    def capture(self, q_chunks, priors, outs=None, dense: bool = False,
                select_only: bool = False) -> torch.cuda.CUDAGraph:
        """Record ``step`` (or ``step_dense``, or only ``select``) for a
        sequence of chunks into one HIP graph; ``replay()`` then reissues every
        kernel with the same arguments and buffers, without the per-call host
        work.  ``outs[i]`` receives chunk i's output (default: the shared
        ``self.out``, which the last chunk leaves).  The library records no
        memset, copy, allocation or synchronisation, so the whole call
        sequence can be captured; inputs must stay at the same addresses
        between replays."""
        if outs is not None and len(outs) != len(q_chunks):
            raise ValueError("outs must give one output per chunk")
        if len(priors) != len(q_chunks):
            raise ValueError("priors must give one offset per chunk")
        lens = [self.dense_lens(p) for p in priors] if dense else None
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i, (q, p) in enumerate(zip(q_chunks, priors)):
                o = outs[i] if outs is not None else None
                if select_only:
                    self.select(q, p)
                elif dense:
                    self.step_dense(q, p, lens[i], out=o)
                else:
                    self.step(q, p, out=o)
        g.ca_dense_lens = lens  # device buffers the graph reads: keep them alive
        return g

    def dense_lens(self, prior: int) -> torch.Tensor:
        n = (prior + self.C) // CA_BLOCK
        return torch.full((self.B, self.H_kv), n, dtype=torch.int32, device=self.k.device)

    def step_dense(self, q_chunk: torch.Tensor, prior: int, lens: torch.Tensor, out=None,
                   stream=None) -> torch.Tensor:
        """Dense baseline: the same attention kernel over every block up to the
        chunk (lens from ``dense_lens``)."""
        out = self.out if out is None else out
        return chunk_attention(q_chunk, self.k, self.v, self.T_dense, lens, [prior] * self.B,
                               [self.C] * self.B, self.scale, out=out, stream=stream)
