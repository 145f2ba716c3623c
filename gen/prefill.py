"""Seeded synthetic input for a whole chunked prefill: one long prompt whose
queries arrive chunk by chunk while its keys and values accumulate.

Chunked prefill (CompactAttention, problem statement of the technical
summaries): the prompt is processed in fixed-size chunks, each attending to
the KV cache accumulated so far, so a mask search and the attention run again
for every chunk over a growing cache.  The pages measure this regime on
LLaMA-3.1-8B at 128K context; with no weights here, the stream stands in for
the attention inputs of one layer.

Recipe (planted structure, so that a block-mask producer has something to
find and different queries of a group agree on it):

* ``PCG64([seed, 0])`` draws K, ``PCG64([seed, 1])`` draws V, both N(0, 1)
  over all L tokens of the prompt; ``PCG64([seed, 3])`` draws one unit
  direction u_g per KV head and the salient KV blocks (each block except the
  sink independently with probability ``salient``); every key row of a
  salient block of KV head g gets ``+ strength * u_g``.
* Queries of chunk c come from ``PCG64([seed, 2, c])``: N(0, 1) plus
  ``strength * u_g`` on every row of the query heads of group g, so the pooled
  scores of salient blocks stand out for every Q-block and head of the group.
* bf16 rounding (round to nearest even) at the end.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict

import numpy as np
import torch

BLOCK = 64


@dataclasses.dataclass
class PrefillStream:
    name: str
    H_q: int
    H_kv: int
    D: int
    L: int            # prompt length (tokens); also the cache capacity
    C: int            # chunk length
    seed: int
    salient: float
    strength: float
    k: torch.Tensor   # CPU bf16 [1, H_kv, L, D]
    v: torch.Tensor
    u: np.ndarray     # float32 [H_kv, D]
    salient_blocks: np.ndarray  # bool [H_kv, L / 64]
    meta: Dict[str, object] = dataclasses.field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def n_chunks(self) -> int:
        return self.L // self.C

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def q_chunk(self, c: int) -> torch.Tensor:
        """CPU bf16 [1, H_q, C, D]: the queries of chunk c."""
        rng = np.random.Generator(np.random.PCG64([self.seed, 2, c]))
        q = rng.standard_normal((1, self.H_q, self.C, self.D), dtype=np.float32)
        q += self.strength * np.repeat(self.u, self.G, axis=0)[None, :, None, :]
        return torch.from_numpy(q).to(torch.bfloat16)


PREFILL_STREAMS = {
    # LLaMA-3.1-8B attention shape, 128K prompt in 64 chunks of 2048 tokens
    "prefill_128k": dict(H_q=32, H_kv=8, D=128, L=131072, C=2048, seed=1006, salient=0.03,
                         strength=2.0),
    # small enough for the float64 oracle on every chunk
    "prefill_small": dict(H_q=8, H_kv=2, D=64, L=2048, C=256, seed=1007, salient=0.1,
                          strength=2.0),
}


def make_prefill_stream(name: str) -> PrefillStream:
    cfg = PREFILL_STREAMS[name]
    H_kv, D, L, seed = cfg["H_kv"], cfg["D"], cfg["L"], cfg["seed"]
    k = np.random.Generator(np.random.PCG64([seed, 0])).standard_normal((1, H_kv, L, D),
                                                                        dtype=np.float32)
    v = np.random.Generator(np.random.PCG64([seed, 1])).standard_normal((1, H_kv, L, D),
                                                                        dtype=np.float32)
    rs = np.random.Generator(np.random.PCG64([seed, 3]))
    u = rs.standard_normal((H_kv, D)).astype(np.float32)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    sal = rs.random((H_kv, L // BLOCK)) < cfg["salient"]
    sal[:, 0] = False
    for g in range(H_kv):
        rows = np.repeat(sal[g], BLOCK)
        k[0, g, rows] += cfg["strength"] * u[g]
    return PrefillStream(name=name, H_q=cfg["H_q"], H_kv=H_kv, D=D, L=L, C=cfg["C"], seed=seed,
                         salient=cfg["salient"], strength=cfg["strength"],
                         k=torch.from_numpy(k).to(torch.bfloat16),
                         v=torch.from_numpy(v).to(torch.bfloat16), u=u, salient_blocks=sal)
