"""Chunk-by-chunk driver of the whole path over a growing KV cache.

Chunked prefill (CompactAttention, problem statement and "Methodology" of the
technical summaries): a long prompt is processed in fixed-size chunks; for
each one the chunk's keys and values are appended to the cache, a
lightweight search makes the per-head block mask over the cache so far, the
union turns it into per-group tables, and zero-copy attention runs the
chunk's queries over the selected blocks.  Every step is a call into the HIP
library; this class only keeps the per-prompt buffers (allocated once, reused
by every chunk) and issues the calls, in order on one stream or, with
``run(..., overlap=True)``, on two streams so that the next chunk's append and
selection fill the compute units that the current chunk's attention leaves
idle near its end.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import (append_kv, append_select_chunk, balanced_workspace_size, block_mask_topk,
               build_union_tables, chunk_attention, chunk_attention_devlen, pool_blocks,
               select_chunk)
from ._lib import CA_BLOCK


class ChunkedPrefill:
    """Per-prompt state: caches [B, H_kv, L, D] (device, bf16 or fp32), pooled
    keys kept across chunks, and the mask / table / output buffers.

    ``step(q_chunk, prior, k_chunk, v_chunk)`` runs one chunk of C tokens at
    absolute offset ``prior``: it appends the chunk's keys and values
    ([B, H_kv, C, D]) to the caches at rows [prior, prior + C), then selects
    and attends.  Without k_chunk / v_chunk the caches must already hold those
    rows.  ``step_dense`` runs the same attention over every block (the dense
    baseline), with the same optional append.  ``balanced`` runs the sparse
    attention through ``chunk_attention(..., balanced=True)``: the union's
    per-group tables differ in length from group to group, and the plan spreads
    that work evenly over the compute units (the workspace is allocated here,
    once).  ``fused_append`` (default) issues a chunk's append and selection as
    one call, ``ca_append_select_chunk``, whose first launch copies the new
    rows and pools them; without it they are ``ca_append_kv`` then
    ``ca_select_chunk``, with the same results bit for bit."""

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, H_q: int, C: int,
                 budget: int, local: int, scale: Optional[float] = None,
                 balanced: bool = False, fused_append: bool = True):
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
        # table sets for the overlapped run: chunk i uses tables[i % 3], so a
        # selection running ahead never writes the tables an attention still reads
        self.tables = ((self.T, self.lens),) + tuple(
            (torch.empty_like(self.T), torch.empty_like(self.lens)) for _ in range(2))
        self._side = None
        self.T_dense = torch.arange(self.NKB, dtype=torch.int32, device=dev).repeat(B * H_kv, 1) \
            .view(B, H_kv, self.NKB)
        self.out = torch.empty((B, H_q, C, D), dtype=k_cache.dtype, device=dev)
        self.balanced = bool(balanced)
        self.fused_append = bool(fused_append)
        # the chunk offset and length in device memory, for the steps whose
        # graph serves every chunk (capture_chunk)
        self.prior_dev = torch.zeros(B, dtype=torch.int32, device=dev)
        self.chunk_dev = torch.full((B,), C, dtype=torch.int32, device=dev)
        self.ws = None
        if self.balanced:
            self.ws = torch.empty(balanced_workspace_size(B, H_q, H_kv, C, D), dtype=torch.uint8,
                                  device=dev)

    def append(self, k_chunk: torch.Tensor, v_chunk: torch.Tensor, prior: int,
               stream=None) -> None:
        """Write the chunk's keys and values [B, H_kv, C, D] into the caches at
        rows [prior, prior + C) (``ca_append_kv``)."""
        append_kv(k_chunk, v_chunk, self.k, self.v, [prior] * self.B, [self.C] * self.B,
                  stream=stream)

    def select(self, q_chunk: torch.Tensor, prior: int, stream=None, tables=None) -> None:
        """Pool the chunk's new key blocks and its queries, make the mask and
        build the union tables (into self.mask and ``tables``, default
        (self.T, self.lens)): the fused ``ca_select_chunk``, four launches."""
        B, C = self.B, self.C
        T, lens = tables if tables is not None else (self.T, self.lens)
        select_chunk(q_chunk, self.k, [prior] * B, [C] * B, self.budget, self.local, self.qbar,
                     self.kbar, self.scores, self.mask, T, lens, stream=stream)

    def append_select(self, k_chunk: torch.Tensor, v_chunk: torch.Tensor,
                      q_chunk: torch.Tensor, prior: int, stream=None, tables=None) -> None:
        """``append`` then ``select``: one ``ca_append_select_chunk`` call (four
        launches) when ``fused_append``, else the two calls (five launches)."""
        if not self.fused_append:
            self.append(k_chunk, v_chunk, prior, stream)
            self.select(q_chunk, prior, stream, tables)
            return
        B, C = self.B, self.C
        T, lens = tables if tables is not None else (self.T, self.lens)
        append_select_chunk(k_chunk, v_chunk, q_chunk, self.k, self.v, [prior] * B, [C] * B,
                            self.budget, self.local, self.qbar, self.kbar, self.scores,
                            self.mask, T, lens, stream=stream)

    def select_separate(self, q_chunk: torch.Tensor, prior: int, stream=None) -> None:
        """The same selection as ``select`` through the separate calls (six
        launches): pooling of keys, pooling of queries, scores and top-k, union."""
        B, C = self.B, self.C
        p_blk, n_blk = prior // CA_BLOCK, (prior + C) // CA_BLOCK
        pool_blocks(self.k, [p_blk] * B, [n_blk] * B, out=self.kbar, stream=stream)
        pool_blocks(q_chunk, [0] * B, [self.NQ] * B, out=self.qbar, stream=stream)
        block_mask_topk(self.qbar, self.kbar, [prior] * B, [C] * B, self.budget, self.local,
                        scores=self.scores, mask=self.mask, stream=stream)
        build_union_tables(self.mask, self.H_kv, [self.NQ] * B, [n_blk] * B, T=self.T,
                           lens=self.lens, stream=stream)

    def attend(self, q_chunk: torch.Tensor, prior: int, out=None, stream=None,
               tables=None) -> torch.Tensor:
        out = self.out if out is None else out
        T, lens = tables if tables is not None else (self.T, self.lens)
        return chunk_attention(q_chunk, self.k, self.v, T, lens, [prior] * self.B,
                               [self.C] * self.B, self.scale, out=out, stream=stream,
                               balanced=self.balanced, workspace=self.ws)

    def step(self, q_chunk: torch.Tensor, prior: int, out=None, stream=None,
             k_chunk: Optional[torch.Tensor] = None,
             v_chunk: Optional[torch.Tensor] = None) -> torch.Tensor:
        if k_chunk is not None:
            self.append_select(k_chunk, v_chunk, q_chunk, prior, stream)
        else:
            self.select(q_chunk, prior, stream)
        return self.attend(q_chunk, prior, out, stream)

    def run(self, q_chunks, priors, outs=None, kv_chunks=None, overlap: bool = True) -> None:
        """A sequence of chunks (``outs[i]``, ``kv_chunks[i]`` as in ``capture``).

        overlap=False issues ``step`` for each chunk on the current stream.
        overlap=True issues the attention on the current stream and each
        chunk's append and selection on a second stream (default priority),
        ahead of the attention: chunk i+1's append, pooling, mask and tables
        run while earlier chunks attend, and take the compute units the
        attention's workgroups leave as they finish.  Events order the two
        streams:
        - chunk i's attention waits for chunk i's selection;
        - chunk i's selection writes tables[i % 3], so it waits for chunk
          i-3's attention, the last reader of that set (the selections may
          run up to two chunks ahead);
        - the appends write cache rows [prior, prior + C), which no earlier
          chunk's attention reads (its keys end at its own prior + C);
        - the pooled keys, queries, scores and mask are used by the selections
          alone, which stay in order on the second stream.
        The current stream waits for the second one at the end.  Every kernel
        gets the same inputs as in the sequential order, so the outputs are
        the same, bit for bit."""
        n = len(q_chunks)
        if outs is not None and len(outs) != n:
            raise ValueError("outs must give one output per chunk")
        if len(priors) != n:
            raise ValueError("priors must give one offset per chunk")
        if kv_chunks is not None and len(kv_chunks) != n:
            raise ValueError("kv_chunks must give one (k, v) pair per chunk")
        if not overlap:
            for i in range(n):
                kc, vc = kv_chunks[i] if kv_chunks is not None else (None, None)
                self.step(q_chunks[i], priors[i], out=outs[i] if outs is not None else None,
                          k_chunk=kc, v_chunk=vc)
            return
        main = torch.cuda.current_stream(self.k.device)
        if self._side is None:
            self._side = torch.cuda.Stream(device=self.k.device)
        side = self._side
        selected = [torch.cuda.Event() for _ in range(n)]
        attended = [torch.cuda.Event() for _ in range(n)]
        side.wait_stream(main)  # inputs written on the current stream come first

        depth = len(self.tables)

        def issue_select(i):
            # the append needs no wait (its rows are past every key an earlier
            # chunk's attention reads), but with fused_append it shares the
            # selection's first launch, which writes tables[i % depth]
            if kv_chunks is not None and not self.fused_append:
                self.append(kv_chunks[i][0], kv_chunks[i][1], priors[i], stream=side)
            if i >= depth:
                side.wait_event(attended[i - depth])
            if kv_chunks is not None and self.fused_append:
                self.append_select(kv_chunks[i][0], kv_chunks[i][1], q_chunks[i], priors[i],
                                   stream=side, tables=self.tables[i % depth])
            else:
                self.select(q_chunks[i], priors[i], stream=side, tables=self.tables[i % depth])
            selected[i].record(side)

        if n > 0:
            issue_select(0)
        for i in range(n):
            main.wait_event(selected[i])
            self.attend(q_chunks[i], priors[i], out=outs[i] if outs is not None else None,
                        stream=main, tables=self.tables[i % depth])
            attended[i].record(main)
            if i + 1 < n:
                issue_select(i + 1)
        main.wait_stream(side)

    def capture(self, q_chunks, priors, outs=None, dense: bool = False,
                select_only: bool = False, kv_chunks=None,
                overlap: bool = False) -> torch.cuda.CUDAGraph:
        """Record ``step`` (or ``step_dense``, or only ``select``) for a
        sequence of chunks into one HIP graph; ``replay()`` then reissues every
        kernel with the same arguments and buffers, without the per-call host
        work.  ``outs[i]`` receives chunk i's output (default: the shared
        ``self.out``, which the last chunk leaves); ``kv_chunks[i]`` =
        (k_chunk, v_chunk) makes chunk i append its keys and values first.
        The library records no memset, copy, allocation or synchronisation, so
        the whole call sequence can be captured; inputs must stay at the same
        addresses between replays.  overlap=True records ``run(...,
        overlap=True)``: the two streams become two branches of the graph,
        joined by the same event edges."""
        if outs is not None and len(outs) != len(q_chunks):
            raise ValueError("outs must give one output per chunk")
        if len(priors) != len(q_chunks):
            raise ValueError("priors must give one offset per chunk")
        if kv_chunks is not None and len(kv_chunks) != len(q_chunks):
            raise ValueError("kv_chunks must give one (k, v) pair per chunk")
        if overlap and (dense or select_only):
            raise ValueError("overlap records the sparse steps only")
        lens = [self.dense_lens(p) for p in priors] if dense else None
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            if overlap:
                self.run(q_chunks, priors, outs=outs, kv_chunks=kv_chunks, overlap=True)
            else:
                self._record_steps(q_chunks, priors, outs, kv_chunks, lens, select_only)
        g.ca_dense_lens = lens  # device buffers the graph reads: keep them alive
        return g

    def _record_steps(self, q_chunks, priors, outs, kv_chunks, lens, select_only):
        for i, (q, p) in enumerate(zip(q_chunks, priors)):
            o = outs[i] if outs is not None else None
            kc, vc = kv_chunks[i] if kv_chunks is not None else (None, None)
            if select_only:
                if kc is not None:
                    self.append_select(kc, vc, q, p)
                else:
                    self.select(q, p)
            elif lens is not None:
                self.step_dense(q, p, lens[i], out=o, k_chunk=kc, v_chunk=vc)
            else:
                self.step(q, p, out=o, k_chunk=kc, v_chunk=vc)

    def set_prior(self, prior: int) -> None:
        """Chunk offset read by ``step_devlen`` and by graphs from ``capture_chunk``."""
        self.prior_dev.fill_(int(prior))

    def step_devlen(self, q_chunk: torch.Tensor, k_chunk: torch.Tensor, v_chunk: torch.Tensor,
                    out=None, stream=None) -> torch.Tensor:
        """``step`` with the chunk's keys and values, taking the chunk offset
        from device memory (``set_prior``): ``ca_append_select_chunk_devlen``
        then ``ca_chunk_attention_devlen``.  No argument depends on the offset,
        so the same calls, captured once, serve every chunk.  Same results as
        ``step`` bit for bit (plain attention, not balanced)."""
        out = self.out if out is None else out
        append_select_chunk(k_chunk, v_chunk, q_chunk, self.k, self.v, self.prior_dev,
                            self.chunk_dev, self.budget, self.local, self.qbar, self.kbar,
                            self.scores, self.mask, self.T, self.lens, stream=stream)
        return chunk_attention_devlen(q_chunk, self.k, self.v, self.T, self.lens, self.prior_dev,
                                      self.chunk_dev, self.scale, out=out, stream=stream)

    def capture_chunk(self, q_buf: torch.Tensor, k_buf: torch.Tensor, v_buf: torch.Tensor,
                      out=None) -> torch.cuda.CUDAGraph:
        """One HIP graph of ``step_devlen`` on fixed input buffers (q_buf
        [B, H_q, C, D], k_buf / v_buf [B, H_kv, C, D]) that serves every chunk of
        every prompt this object holds: write the chunk's queries, keys and
        values into the buffers and its offset with ``set_prior``, then replay."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step_devlen(q_buf, k_buf, v_buf, out=out)
        return g

    def dense_lens(self, prior: int) -> torch.Tensor:
        n = (prior + self.C) // CA_BLOCK
        return torch.full((self.B, self.H_kv), n, dtype=torch.int32, device=self.k.device)

    def step_dense(self, q_chunk: torch.Tensor, prior: int, lens: torch.Tensor, out=None,
                   stream=None, k_chunk: Optional[torch.Tensor] = None,
                   v_chunk: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Dense baseline: the same attention kernel over every block up to the
        chunk (lens from ``dense_lens``), after the same optional append."""
        if k_chunk is not None:
            self.append(k_chunk, v_chunk, prior, stream)
        out = self.out if out is None else out
        return chunk_attention(q_chunk, self.k, self.v, self.T_dense, lens, [prior] * self.B,
                               [self.C] * self.B, self.scale, out=out, stream=stream)
