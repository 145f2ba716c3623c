"""The append step of chunked prefill, written as its definition.

CompactAttention, problem statement of the technical summaries: a long prompt
is processed in chunks, each attending to the cache accumulated so far and,
causally, to itself; so before a chunk attends, its own keys and values are
written into the cache after the prior tokens:

    K_cache[b, g, prior[b] + i, :] = K_new[b, g, i, :]    for i < chunk[b]
    (V likewise; every other row of the cache keeps its value).

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def append_kv_ref(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray,
                  v_new: np.ndarray, prior: Sequence[int], chunk: Sequence[int]
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """k_cache, v_cache [B,H_kv,L,D]; k_new, v_new [B,H_kv,C_max,D].  Returns new
    caches (the inputs are not modified)."""
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    for b in range(k_cache.shape[0]):
        P, C = int(prior[b]), int(chunk[b])
        for i in range(C):
            k_out[b, :, P + i] = k_new[b, :, i]
            v_out[b, :, P + i] = v_new[b, :, i]
    return k_out, v_out
