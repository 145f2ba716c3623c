// Internal interface between the C-ABI layer (capi.hip) and the kernel files.
// Everything here is validated by the caller before a launcher is invoked.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "compact_attn.h"

namespace ca {

// Per-sequence extents of the block mask (union builder).
struct UnionExtents {
  int32_t nq[CA_MAX_BATCH];   // Q-block rows of the chunk
  int32_t nkb[CA_MAX_BATCH];  // KV blocks of the sequence (prior + chunk)
};

// Per-sequence lengths of one chunk-attention call, plus the order in which
// sequences are handed to workgroups (longest first, so the longest work
// starts earliest).
struct SeqInfo {
  int32_t prior[CA_MAX_BATCH];
  int32_t chunk[CA_MAX_BATCH];
  int32_t order[CA_MAX_BATCH];
};

// Per-sequence block ranges [begin, end) of a pooling call.
struct BlockRange {
  int32_t begin[CA_MAX_BATCH];
  int32_t end[CA_MAX_BATCH];
};

// Balance plan limits: pieces per (b, g, tile), and compute units the plan
// spreads pieces over (the device's count, up to this many).
constexpr int kMaxPieces = 8;
constexpr int kPlanMaxSlots = 1024;
constexpr int kPlanMaxBlocks = 1 << 24;  // NKB_max the plan's 32-bit piece arithmetic allows

struct AttnParams {
  int H_q, H_kv, G;     // heads; G = H_q / H_kv query heads per KV head
  int C_max;            // rows of Q/O per head
  int64_t L;            // cache capacity (tokens) per (b, KV head)
  int NKB_max;          // row length of T
  float scale;          // softmax scale on Q.K
  float scale_log2;     // scale * log2(e)
  int n_t;              // workgroups per (b, g) pseudo-request
  int xcd;              // 1: keep each pseudo-request's workgroups on one XCD
  int row_tables;       // 0: T[b,g] (union); 1: T[b,h,Q-block] (per-Q-block lists)
  int NQ_max;           // Q-blocks per head in the per-Q-block table layout
  int waves;            // bf16 union tables: waves per workgroup (4 or 8)
  int n_split;          // split-KV: table ranges per (b, g) (1: no split)
  int64_t rows_total;   // B * H_q * C_max (split-KV partial layout)
  int cus;              // compute units of the device (launch shape choices only)
  // balance plan (bf16 planned pieces): plan_items[0] = number of pieces, then
  // one int4 (b * H_kv + g, tile, piece k, pieces n) per piece from int 4 on;
  // plan_pieces[(b * H_kv + g) * n_t + tile] = n
  const int32_t* plan_items;
  const int32_t* plan_pieces;
};

hipError_t launch_union_tables(const uint8_t* mask, int B, int H_q, int H_kv, int NQ_max,
                               int NKB_max, const UnionExtents& ext, int32_t* T,
                               int32_t* len, hipStream_t stream);

hipError_t launch_check_tables(const int32_t* T, const int32_t* len, int n_bg, int H_kv,
                               int NKB_max, const UnionExtents& ext, int32_t* row_bad,
                               hipStream_t stream);
hipError_t launch_tables_to_csr(const int32_t* T, const int32_t* len, int n_bg, int NKB_max,
                                int64_t pages, int32_t* kv_indptr, int32_t* kv_indices,
                                hipStream_t stream);

// bf16 path on the matrix cores; D in {64, 128}.
hipError_t launch_chunk_attn_bf16(const void* Q, const void* K, const void* V,
                                  const int32_t* T, const int32_t* len, void* O, float* lse,
                                  int B, int D, const AttnParams& p, const SeqInfo& seq,
                                  hipStream_t stream);

// bf16 path with each (b, g) table cut into p.n_split ranges: partial
// results in part_o (float [n_split, B*H_q*C_max, D]) and part_ml (float
// [n_split, B*H_q*C_max, 2]: running max, denominator), then a combine kernel
// writes O and lse.
hipError_t launch_chunk_attn_bf16_split(const void* Q, const void* K, const void* V,
                                        const int32_t* T, const int32_t* len, void* O,
                                        float* lse, int B, int D, const AttnParams& p,
                                        const SeqInfo& seq, float* part_o, float* part_ml,
                                        hipStream_t stream);

// bf16 path with a balance plan: a planning kernel cuts the (b, g, tile)
// workgroups whose table walks are longest into pieces so that the pieces
// spread evenly over p.cus compute units (longest first), writes the plan to
// plan (p.plan_items / p.plan_pieces point into it), then the pieces run
// (8-wave workgroups) and a merge combines the cut tiles' partials.
hipError_t launch_chunk_attn_bf16_balanced(const void* Q, const void* K, const void* V,
                                           const int32_t* T, const int32_t* len, void* O,
                                           float* lse, int B, int D, const AttnParams& p,
                                           const SeqInfo& seq, float* part_o, float* part_ml,
                                           hipStream_t stream);

// fp32 path on the vector ALUs; D in {64, 128}.
hipError_t launch_chunk_attn_f32(const float* Q, const float* K, const float* V,
                                 const int32_t* T, const int32_t* len, float* O, float* lse,
                                 int B, int D, const AttnParams& p, const SeqInfo& seq,
                                 hipStream_t stream);
// fp32 split-KV: partials of p.n_split table ranges, then the merge.
hipError_t launch_chunk_attn_f32_split(const float* Q, const float* K, const float* V,
                                       const int32_t* T, const int32_t* len, float* O,
                                       float* lse, int B, int D, const AttnParams& p,
                                       const SeqInfo& seq, float* part_o, float* part_ml,
                                       hipStream_t stream);
// Merge of split-KV partials (part_o unnormalised fp32 [n_split, rows, D],
// part_ml (running max, denominator) per row) into O (bf16, or fp32 when
// f32_out) and lse.
hipError_t launch_split_combine(const float* part_o, const float* part_ml, int D, bool f32_out,
                                void* O, float* lse, const AttnParams& p, const SeqInfo& seq,
                                hipStream_t stream);

// Explicit KV compaction (baseline); esz = element size in bytes.
hipError_t launch_compact_kv(const void* K, const void* V, const int32_t* T, const int32_t* len,
                             int NKB_max, int B, int H_kv, int64_t L, int D, int esz,
                             const SeqInfo& seq, void* Ko, void* Vo, int32_t* To,
                             hipStream_t stream);

// Block-mask producer: mean pooling of 64-row blocks (esz = 2: bf16, 4: fp32).
hipError_t launch_pool_blocks(const void* X, int esz, int B, int H, int64_t R, int D,
                              const BlockRange& rng, int max_span, float* out, int NB_out,
                              hipStream_t stream);

// Block-mask producer: pooled scores, then per-row top-k selection.
hipError_t launch_block_mask(const float* qbar, const float* kbar, int B, int H_q, int H_kv,
                             int NQ_max, int NKB_max, int D, const SeqInfo& seq, int max_pblk,
                             int budget, int local, float* scores, uint8_t* mask,
                             hipStream_t stream);

}  // namespace ca
