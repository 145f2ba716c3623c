"""CPU oracle for the CompactAttention chunked-prefill hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call anything in this package.
The product path (the HIP library and its Python binding) never does, and
this package imports nothing from it: the two share no code, only the seeded
inputs of the ``gen`` package.

Contents (each function cites the passage it follows):

* ``union_tables_ref``   -- Block-Union KV selection: Q-block union, then
  intra-group union, giving the minimal coverage-preserving per-group block
  table T[b,g] and its length.  Pinned by brute force, a hand-worked fixture,
  set invariants and special cases.
* ``chunk_attention_ref`` -- softmax attention of a chunk's queries over the
  keys of the blocks in T[b,g], causal inside the current chunk.  Pinned by
  torch's SDPA on the dense special case, brute-force loops, closed forms
  (K=0, one-hot V, V=1, single admissible key), shift invariance and the
  empty-set convention.
* ``chunk_attention_dense_masked_ref`` -- the same result computed as dense
  attention over all cached keys with a -inf mask (second formulation).
* ``tables_to_csr_ref`` -- the (kv_indptr, kv_indices) view of the tables.
* ``check_tables_ref`` -- the table contract attention relies on (range,
  strict ascent, -1 padding), checked row by row.  Pinned by the tables of
  ``union_tables_ref`` (all rows pass) and by planted single violations,
  each giving exactly its own flag.
* ``append_kv_ref`` -- the append step of chunked prefill: a chunk's keys and
  values written into the cache after the prior tokens.  Pinned by a
  hand-worked case and by rebuilding a whole prompt chunk by chunk, in any
  order.
* ``compact_kv_ref`` -- explicit KV compaction (the copy zero-copy execution
  avoids): selected prior blocks packed to end where the chunk starts.  Pinned
  by a hand-worked case and by the invariant that attention over the
  compacted cache equals attention over the original one.
* ``sparse_attention_ref`` -- block-sparse-kernel execution of the mask (each
  Q-block of each head attends its own mask row, no union).  Pinned by
  brute-force loops, by the reduction to the union attention when every row
  of a group is the same, and by the dense special case.
* ``producer_mask_ref`` (with ``pool_blocks_ref``, ``block_scores_ref``,
  ``topk_mask_ref``) -- a training-free block-mask producer: mean-pooled
  Q-block . mean-pooled K-block scores, per-row top-k plus sink, local window
  and the causal block triangle.  Pinned by closed forms of the pooling, brute
  force on the scores and sort-based brute force on the selection.

Float work is float64 throughout; outputs are float32.
"""
from .union_ref import check_tables_ref, tables_to_csr_ref, union_tables_ref  # noqa: F401
from .attention_ref import (  # noqa: F401
    BLOCK,
    admissible_keys,
    chunk_attention_dense_masked_ref,
    chunk_attention_ref,
    chunk_attention_rows_ref,
)
from .append_ref import append_kv_ref  # noqa: F401
from .compact_ref import compact_kv_ref  # noqa: F401
from .sparse_ref import sparse_attention_ref, sparse_attention_rows_ref  # noqa: F401
from .producer_ref import (block_scores_ref, pool_blocks_ref, producer_mask_ref,  # noqa: F401
                           topk_mask_ref)
