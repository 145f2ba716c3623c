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

// Balanced attention limits: slots (one workgroup per compute unit, the
// device's count up to this many) and the least work per slot before tiles
// are cut.  Calls with more tiles than slots, or with tiles * NKB_max past
// 2^31 - 1 (the plan's 32-bit sums), run the plain kernel instead.
constexpr int kPlanMaxSlots = 1024;
constexpr int kBalMinShare = 32;
constexpr int kBalJobCost = 12;  // work units a job costs on its own, in the plan

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
  // balanced attention: tiles of the plan (B * H_kv * n_t), partial tiles the
  // workspace holds, and the plan's part numbering (bal_units + 1 ints: parts
  // of the cut tiles before tile i, then the total), written by the attention
  // kernel and read by the merge
  int bal_units;
  int bal_parts;
  int32_t* bal_pre;
  // device-length calls: prior and chunk lengths read from device int32 [B]
  // arrays (nullptr: the host values in SeqInfo)
  const int32_t* dev_prior;
  const int32_t* dev_chunk;
  // stamped calls (bf16 union tables, no split): per-workgroup timing words,
  // kStampWords per workgroup (nullptr: none written)
  uint32_t* stamps;
};

// Timing words per workgroup of a stamped call: start of the 100 MHz
// real-time counter (low 32 bits), its ticks until the epilogue, the
// shader-clock cycles over the same span, and the hardware ids (XCC in bits
// 0..3, the HW_ID register's CU / SH / SE fields in bits 8..15).
constexpr int kStampWords = 4;

// Prior and chunk length of sequence b in a kernel.  Host-length calls pass
// values the host has already checked.  Device-length calls read them from
// device memory and check them here against the call's limits: a sequence
// whose lengths are negative, not multiples of 64, a chunk past C_max, or a
// total past the cache capacity or the table length runs as an empty chunk
// (its rows give O = 0 and lse = -inf; nothing else is read).
__device__ __forceinline__ void seq_lengths(const AttnParams& p, const SeqInfo& seq, int b,
                                            int& P, int& C) {
  if (p.dev_prior == nullptr) {
    P = seq.prior[b];
    C = seq.chunk[b];
    return;
  }
  const int P_ = p.dev_prior[b];
  const int C_ = p.dev_chunk[b];
  const int64_t cap = p.L < 64 * static_cast<int64_t>(p.NKB_max)
                          ? p.L : 64 * static_cast<int64_t>(p.NKB_max);
  const bool ok = P_ >= 0 && C_ >= 0 && ((P_ | C_) & 63) == 0 && C_ <= p.C_max &&
                  static_cast<int64_t>(P_) + C_ <= cap;
  P = ok ? P_ : 0;
  C = ok ? C_ : 0;
}

// Device address of the library's static scratch array (CA_STATIC_SCRATCH_BYTES)
// on the current device, looked up once per device; nullptr, with the HIP
// error in *err, if the lookup fails.
void* static_scratch_address(hipError_t* err);

// dev_nq / dev_nkb: device int32 [B] extents (device-length call), or nullptr
// to use ext.  cus: compute units of the device (how finely the OR step is
// spread when there are few pseudo-requests; T then also holds intermediate
// bitmap words during the call).
hipError_t launch_union_tables(const uint8_t* mask, int B, int H_q, int H_kv, int NQ_max,
                               int NKB_max, const UnionExtents& ext, const int32_t* dev_nq,
                               const int32_t* dev_nkb, int32_t* T, int32_t* len, int cus,
                               hipStream_t stream);

// Compaction of union bitmaps parked at the tail of each T row (n_rep copies
// of ceil(NKB_max / 32) words, ORed together; n_rep * words <= NKB_max) into
// the rows themselves and len, one workgroup per row.
hipError_t launch_union_compact(int n_bg, int NKB_max, int n_rep, int32_t* T, int32_t* len,
                                hipStream_t stream);

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

// bf16 path, balanced: one 8-wave workgroup per slot (slots <= kPlanMaxSlots,
// the device's compute units); each derives the plan from the table lengths
// and runs its pieces; the pieces of cut tiles write partials (part_o: float
// [p.bal_parts, 256, D]; part_ml: float [p.bal_parts, 256, 2]) that a merge
// kernel then combines (p.bal_pre: the part numbering, p.bal_units + 1 ints).
// p.n_t = tiles of 8 waves per (b, g); p.bal_units <= slots.
hipError_t launch_chunk_attn_bf16_balanced(const void* Q, const void* K, const void* V,
                                           const int32_t* T, const int32_t* len, void* O,
                                           float* lse, int D, const AttnParams& p,
                                           const SeqInfo& seq, float* part_o, float* part_ml,
                                           int slots, hipStream_t stream);

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

// Append of a chunk's K/V ([B, H_kv, C_max, D], rows [0, chunk)) to the cache
// rows [prior, prior + chunk); esz = element size in bytes.
hipError_t launch_append_kv(const void* k_new, const void* v_new, int B, int H_kv, int C_max,
                            int64_t L, int D, int esz, const SeqInfo& seq, void* k_cache,
                            void* v_cache, hipStream_t stream);

// Explicit KV compaction (baseline); esz = element size in bytes.
hipError_t launch_compact_kv(const void* K, const void* V, const int32_t* T, const int32_t* len,
                             int NKB_max, int B, int H_kv, int64_t L, int D, int esz,
                             const SeqInfo& seq, void* Ko, void* Vo, int32_t* To,
                             hipStream_t stream);

// Block-mask producer: mean pooling of 64-row blocks (esz = 2: bf16, 4: fp32).
hipError_t launch_pool_blocks(const void* X, int esz, int B, int H, int64_t R, int D,
                              const BlockRange& rng, int max_span, float* out, int NB_out,
                              hipStream_t stream);

// A chunk's whole selection step in four launches: pool its new key blocks
// and its Q-blocks (clearing the union bitmap words of T), the scores, the
// top-k mask with the union bits ORed in, the union compaction (esz = 2:
// bf16, 4: fp32 for Q and K).
// With `app`, the first launch also appends the chunk's keys and values to
// the caches (K is then not read: the key blocks are pooled from app->k_new).
struct AppendSrc {
  const void* k_new;  // [B, H_kv, C_max, D], the chunk's rows
  const void* v_new;
  void* k_cache;      // [B, H_kv, L, D], written at rows [prior, prior + chunk)
  void* v_cache;
};
// Device-length selection calls: prior and chunk lengths in device int32 [B]
// arrays, checked by the kernels against chunk_cap and total_cap (prior and
// total_cap = min(L, 64 * NKB_max), chunk_cap = min(C_max, 64 * NQ_max)); a
// default-constructed SelLens (prior == nullptr) means the host values in
// SeqInfo.  With device lengths, max_nq and max_pblk are the bounds those caps
// allow, so the grids do not depend on the lengths.
struct SelLens {
  const int32_t* prior = nullptr;
  const int32_t* chunk = nullptr;
  int chunk_cap = 0;
  int64_t total_cap = 0;
};
hipError_t launch_select_chunk(const void* Q, const void* K, int esz, int B, int H_q, int H_kv,
                               int C_max, int64_t L, int D, const SeqInfo& seq, int max_nq,
                               int max_pblk, int budget, int local, float* qbar, int NQ_max,
                               float* kbar, int NKB_max, float* scores, uint8_t* mask,
                               int32_t* T, int32_t* len, const AppendSrc* app, const SelLens& dl,
                               hipStream_t stream);

// Block-mask producer: pooled scores, then per-row top-k selection.
hipError_t launch_block_mask(const float* qbar, const float* kbar, int B, int H_q, int H_kv,
                             int NQ_max, int NKB_max, int D, const SeqInfo& seq, int max_pblk,
                             int budget, int local, float* scores, uint8_t* mask,
                             hipStream_t stream);

}  // namespace ca
