/*
 * compact_attn.h -- C ABI of the CompactAttention chunked-prefill hot path
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (CompactAttention: Accelerating Chunked Prefill with Block-Union
 * KV Selection; "Methodology" of the technical summaries and the abstract) has
 * two stages, exported here as two separate calls so that *which* KV blocks
 * are selected stays decoupled from *how* they are executed:
 *
 *   1. Selection.  A per-head 2D block mask (Q-block x KV-block) becomes one KV
 *      block table per (sequence, KV head): the union over the chunk's Q-blocks
 *      and over the query heads that share the KV head.  The table is the
 *      minimal one that keeps every selected block.       -> ca_build_union_tables
 *   2. Execution.  Dense attention for the chunk's queries reads the blocks in
 *      the table in place from a KV-head-major [B, H_kv, L, D] cache, where each
 *      (batch, KV head, block) triple is one contiguous region; nothing is
 *      gathered or compacted.                               -> ca_chunk_attention
 *
 * The tables can also be handed over as paged metadata (kv_indptr /
 * kv_indices), the form the pages name for the paged dense kernel.
 *                                                          -> ca_tables_to_csr
 *
 * Conventions shared by every call
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     never allocates or frees device memory and keeps no mutable state,
 *     except the static device array of ca_chunk_attention_split_noalloc.
 *   - Device pointers point to device memory of the current HIP device.  Host
 *     arrays are read during the call only.
 *   - Asynchrony: every call enqueues its kernels on `stream` (0 = the null
 *     stream) and returns without synchronising.  Argument errors are found
 *     on the host before anything is enqueued; the return value then says
 *     which, and no device memory is touched.
 *   - Block size: 64 tokens for both the KV block and the Q-block.
 *   - Errors: a call returns CA_OK or the first error found; see
 *     ca_status_string.  CA_ERR_HIP means a HIP launch reported an error (the
 *     HIP error string is available from ca_last_hip_error).
 */
#ifndef COMPACT_ATTN_H
#define COMPACT_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef CA_EXPORT
#define CA_EXPORT __attribute__((visibility("default")))
#endif

#define CA_BLOCK 64      /* tokens per KV block and per Q-block */
#define CA_MAX_BATCH 128 /* sequences per call */
#define CA_MAX_SPLITS 16 /* split-KV ranges per (sequence, KV head) */
/* Bytes of the library's static device array behind
 * ca_chunk_attention_split_noalloc: 64 MiB, one copy per device. */
#define CA_STATIC_SCRATCH_BYTES (64u << 20)

typedef enum {
  CA_OK = 0,
  CA_ERR_NULL = 1,        /* a required pointer is NULL */
  CA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  CA_ERR_DTYPE = 3,       /* unknown element type */
  CA_ERR_UNSUPPORTED = 4, /* valid request this library does not run (see each call) */
  CA_ERR_HIP = 5,         /* the HIP runtime reported an error */
  CA_ERR_TOO_LARGE = 6    /* needs more than CA_STATIC_SCRATCH_BYTES (no-alloc call only) */
} ca_status;

typedef enum { CA_F32 = 0, CA_BF16 = 1 } ca_dtype;

/*
 * ca_build_union_tables -- Block-Union KV selection (selection stage: Q-block
 * union, then intra-group union, giving the minimal coverage-preserving
 * per-group table T[b,g]).
 *
 *   T[b,g] = ascending { kb < n_kv_blocks[b] : some head h of group g and some
 *            Q-block qb < n_q_blocks[b] have mask[b,h,qb,kb] != 0 }
 *
 * mask        device uint8 [B, H_q, NQ_max, NKB_max], row-major.  Any nonzero
 *             byte selects.  Cells with qb >= n_q_blocks[b] or
 *             kb >= n_kv_blocks[b] are ignored.
 * B           1..CA_MAX_BATCH sequences.
 * H_q, H_kv   query heads and KV heads; H_q % H_kv == 0.  Query head h belongs
 *             to group h / (H_q / H_kv).
 * NQ_max      Q-block rows per head in `mask` (>= 1).
 * NKB_max     KV-block columns in `mask`, and the row length of T (1..524288).
 * n_q_blocks  host int32 [B], 0 <= n_q_blocks[b] <= NQ_max.
 * n_kv_blocks host int32 [B], 0 <= n_kv_blocks[b] <= NKB_max.
 * T           device int32 [B, H_kv, NKB_max] (out): strictly ascending block
 *             ids, then -1 up to NKB_max.
 * len         device int32 [B, H_kv] (out): number of valid entries of T[b,g].
 * Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_HIP.
 *
 * Per-(head, Q-block) lists for ca_chunk_attention_rows come from the same
 * call on the same mask bytes viewed as [B, H_q*NQ_max, 1, NKB_max] (H_q and
 * H_kv both set to H_q*NQ_max, NQ_max = 1, n_q_blocks[b] = 1): each "group"
 * is then a single mask row, and its union is that row's set of blocks.
 */
CA_EXPORT ca_status ca_build_union_tables(const uint8_t* mask, int B, int H_q, int H_kv, int NQ_max,
                                int NKB_max, const int32_t* n_q_blocks,
                                const int32_t* n_kv_blocks, int32_t* T, int32_t* len,
                                hipStream_t stream);

/*
 * ca_build_union_tables_devlen -- ca_build_union_tables with the per-sequence
 * extents in device memory, so that a captured HIP graph can be replayed for
 * a new chunk after only those device values change.
 *
 * n_q_blocks, n_kv_blocks  device int32 [B], 4-byte aligned (else
 *             CA_ERR_UNSUPPORTED), read by the kernel when it runs.  A
 *             sequence with n_q_blocks[b] outside [0, NQ_max] or n_kv_blocks[b]
 *             outside [0, NKB_max] gets an empty table (len 0, T all -1).
 * Every other argument, the result and the errors as for ca_build_union_tables.
 */
CA_EXPORT ca_status ca_build_union_tables_devlen(const uint8_t* mask, int B, int H_q, int H_kv,
                                       int NQ_max, int NKB_max, const int32_t* n_q_blocks,
                                       const int32_t* n_kv_blocks, int32_t* T, int32_t* len,
                                       hipStream_t stream);

/*
 * ca_chunk_attention -- zero-copy paged chunk attention (execution stage).
 *
 * For sequence b, query head h (group g = h / (H_q/H_kv)) and chunk row
 * i < chunk_len[b] at absolute position p = prior_len[b] + i:
 *
 *   A    = { t : T[b,g,j] == t/64 for some j < len[b,g],  t <= p }
 *   O    = softmax_{t in A}( scale * Q[b,h,i,:] . K[b,g,t,:] ) @ V[b,g,A,:]
 *   lse  = log sum_{t in A} exp(scale * Q[b,h,i,:] . K[b,g,t,:])   (natural log)
 *
 * The chunk's own keys/values must already be in the cache at rows
 * [prior_len[b], prior_len[b] + chunk_len[b]).  Key/value rows outside the
 * blocks of T[b,g] are never read.  An empty A gives O = 0, lse = -inf; rows
 * chunk_len[b] <= i < C_max give O = 0, lse = -inf.
 *
 * Q, O        device [B, H_q, C_max, D], element type `dtype`, row-major, 16-byte
 *             aligned.  O is fully written.
 * K_cache,    device [B, H_kv, L, D], element type `dtype`, KV-head-major,
 * V_cache     16-byte aligned.
 * T, len      device, as produced by ca_build_union_tables: T int32
 *             [B, H_kv, NKB_max] with strictly ascending entries, len int32
 *             [B, H_kv].  Entries outside [0, n_kv_blocks[b]) and len values
 *             outside [0, NKB_max] are clamped away, never dereferenced.
 * prior_len,  host int32 [B]: cached tokens before the chunk, and chunk tokens.
 * chunk_len   Both multiples of 64 (else CA_ERR_UNSUPPORTED);
 *             0 <= chunk_len[b] <= C_max; prior_len[b] + chunk_len[b] <= L and
 *             <= 64 * NKB_max.
 * B           1..CA_MAX_BATCH.  H_q % H_kv == 0.
 * D           head dim: 64 or 128 (else CA_ERR_UNSUPPORTED).
 * block       must be 64 (else CA_ERR_UNSUPPORTED).
 * scale       softmax scale applied to Q.K (1/sqrt(D) in the usual case); > 0.
 * dtype       CA_BF16: bf16 in/out, fp32 accumulation on the matrix cores,
 *             probabilities rounded to bf16 for the P.V product.  Requires
 *             L * D * 2 < 2^32 (a 4 GiB cache slice per (b, g); else
 *             CA_ERR_UNSUPPORTED).
 *             CA_F32:  fp32 in/out and fp32 arithmetic throughout.
 * lse         device float [B, H_q, C_max] (out) or NULL.
 * Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_DTYPE, CA_ERR_UNSUPPORTED, CA_ERR_HIP.
 */
CA_EXPORT ca_status ca_chunk_attention(const void* Q, const void* K_cache, const void* V_cache,
                             const int32_t* T, const int32_t* len, int NKB_max,
                             const int32_t* prior_len, const int32_t* chunk_len, int B,
                             int H_q, int H_kv, int C_max, int64_t L, int D, int block,
                             float scale, ca_dtype dtype, void* O, float* lse,
                             hipStream_t stream);

/*
 * ca_chunk_attention_devlen -- ca_chunk_attention with prior_len and
 * chunk_len in device memory (CompactAttention, execution stage: the tables
 * and the per-request lengths travel to the paged dense kernel as device
 * metadata).  The grid depends only on B, H_q, H_kv and C_max, so one
 * captured HIP graph serves every chunk offset: between replays only the
 * device lengths (and the inputs' contents) change.
 *
 * prior_len,  device int32 [B], 4-byte aligned (else CA_ERR_UNSUPPORTED),
 * chunk_len   read by the kernels when they run.  The conditions of
 *             ca_chunk_attention (multiples of 64, chunk_len <= C_max,
 *             prior_len + chunk_len <= L and <= 64 * NKB_max) are checked
 *             there: a sequence that breaks them is computed as an empty chunk
 *             (every row O = 0, lse = -inf) and reads nothing from the cache.
 * Sequences run in index order (the host does not see the lengths, so the
 * longest-first order of ca_chunk_attention is not applied).  With valid
 * lengths the result equals ca_chunk_attention's bit for bit.
 * Every other argument and the errors as for ca_chunk_attention.
 */
CA_EXPORT ca_status ca_chunk_attention_devlen(const void* Q, const void* K_cache,
                                    const void* V_cache, const int32_t* T, const int32_t* len,
                                    int NKB_max, const int32_t* prior_len,
                                    const int32_t* chunk_len, int B, int H_q, int H_kv,
                                    int C_max, int64_t L, int D, int block, float scale,
                                    ca_dtype dtype, void* O, float* lse, hipStream_t stream);

/*
 * ca_chunk_attention_stamped -- ca_chunk_attention (bf16) that also records,
 * per workgroup, when it ran and at what shader clock: a measurement aid for
 * the execution stage's kernel (how long each workgroup's table walk takes,
 * on which XCD, at which clock).  Same result as ca_chunk_attention, bit for
 * bit.
 *
 * stamps          device uint32 [max_workgroups, 4] (out), 4-byte aligned.
 *                 Record w: [0] start of the 100 MHz real-time counter (low 32
 *                 bits); [1] its ticks until the workgroup's epilogue; [2]
 *                 shader-clock cycles over the same span (so the clock is
 *                 [2] / [1] * 100 MHz); [3] XCC id in bits 0..3, the HW_ID
 *                 register's CU / SH / SE fields in bits 8..15.
 * max_workgroups  records the buffer holds; stamps may be NULL with
 *                 max_workgroups = 0, to learn the count.
 * n_workgroups    host int (out): the workgroups the call launches (set even
 *                 when the buffer is too small, which gives CA_ERR_SHAPE and
 *                 launches nothing).
 * dtype           CA_BF16 only (else CA_ERR_UNSUPPORTED).
 * Other arguments, layouts and errors as for ca_chunk_attention.
 */
CA_EXPORT ca_status ca_chunk_attention_stamped(const void* Q, const void* K_cache,
                                     const void* V_cache, const int32_t* T, const int32_t* len,
                                     int NKB_max, const int32_t* prior_len,
                                     const int32_t* chunk_len, int B, int H_q, int H_kv,
                                     int C_max, int64_t L, int D, int block, float scale,
                                     ca_dtype dtype, void* O, float* lse, uint32_t* stamps,
                                     int max_workgroups, int* n_workgroups, hipStream_t stream);

/*
 * ca_chunk_attention_split -- ca_chunk_attention with each (b, g) table cut
 * into n_splits contiguous ranges processed by separate workgroups, then
 * merged.  For shapes with few (sequence, KV head) pairs, such as one GPU's
 * share of the KV heads under tensor parallelism (H_kv = 1): the same result
 * (the same admissible keys and the same softmax), up to the rounding of the
 * merge.  Split s keeps an unnormalised partial output a_s, its running max
 * m_s and denominator l_s; with M = max_s m_s and w_s = exp(scale*(m_s - M)),
 *   O = sum_s w_s a_s / sum_s w_s l_s,   lse = scale*M + log(sum_s w_s l_s),
 * The pages do not describe splitting one table over several workers; this
 * is the usual merge of partial softmax results, exact up to rounding.
 *
 * n_splits   1..CA_MAX_SPLITS (else CA_ERR_SHAPE); 1 is ca_chunk_attention
 *            itself (workspace unused).
 * workspace  device memory owned by the caller, 16-byte aligned, at least
 *            ca_chunk_attention_workspace_size(B, H_q, C_max, D, n_splits)
 *            bytes (else CA_ERR_SHAPE); NULL only when n_splits == 1.
 * dtype      CA_BF16 or CA_F32; the partials and the merge are fp32 for both.
 * Other arguments, layouts and errors as for ca_chunk_attention.  Calls that
 * share one workspace must be ordered on one stream.
 */
CA_EXPORT ca_status ca_chunk_attention_split(const void* Q, const void* K_cache,
                                   const void* V_cache, const int32_t* T, const int32_t* len,
                                   int NKB_max, const int32_t* prior_len,
                                   const int32_t* chunk_len, int B, int H_q, int H_kv,
                                   int C_max, int64_t L, int D, int block, float scale,
                                   ca_dtype dtype, int n_splits, void* workspace,
                                   size_t workspace_bytes, void* O, float* lse,
                                   hipStream_t stream);

/* Bytes of workspace ca_chunk_attention_split needs: n_splits * B * H_q *
 * C_max * (D + 2) * 4 (partial outputs, running maxima, denominators); 0 for
 * n_splits < 2 or nonpositive sizes. */
CA_EXPORT size_t ca_chunk_attention_workspace_size(int B, int H_q, int C_max, int D,
                                         int n_splits);

/*
 * ca_chunk_attention_split_noalloc -- ca_chunk_attention_split for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The split partials live in
 * a static device array of CA_STATIC_SCRATCH_BYTES inside the library (one
 * copy per device, held until the process ends) instead of a caller
 * workspace; the caller still passes every input and output.  The call makes
 * no hipMalloc, hipFree or other allocating call.  The array's device address
 * is looked up (hipGetSymbolAddress) on the first call on each device, after
 * the arguments have been checked.
 *
 * Same kernels, arguments, layouts and result as ca_chunk_attention_split
 * with n_splits, bit for bit.  n_splits == 1 runs ca_chunk_attention (the
 * array is not used).
 * Limit: ca_chunk_attention_workspace_size(B, H_q, C_max, D, n_splits) must
 * not exceed CA_STATIC_SCRATCH_BYTES, else CA_ERR_TOO_LARGE (nothing is
 * enqueued).  For example one GPU's tensor-parallel share of a 2048-token
 * chunk (H_q = 4, D = 128) at n_splits = 8 needs 32.5 MiB.
 * Every call on one device shares that device's array and leaves its partials
 * there: calls that overlap on one device (different streams, or threads
 * without ordering) race and give wrong results; order them on one stream.
 * Nothing in the array needs to start at zero.
 * Errors: those of ca_chunk_attention_split, and CA_ERR_TOO_LARGE.
 */
CA_EXPORT ca_status ca_chunk_attention_split_noalloc(const void* Q, const void* K_cache,
                                           const void* V_cache, const int32_t* T,
                                           const int32_t* len, int NKB_max,
                                           const int32_t* prior_len, const int32_t* chunk_len,
                                           int B, int H_q, int H_kv, int C_max, int64_t L,
                                           int D, int block, float scale, ca_dtype dtype,
                                           int n_splits, void* O, float* lse,
                                           hipStream_t stream);

/*
 * ca_chunk_attention_balanced -- ca_chunk_attention with the work spread
 * evenly over the compute units when the tables are uneven: tables of
 * different lengths across (sequence, KV head) pairs, as a mask producer's
 * union gives from chunk to chunk (CompactAttention, selection stage: T[b,g]
 * holds what each group's union selected, so lengths differ by group), and
 * the causal part, which grows along the chunk.  The pages do not describe
 * how work is scheduled; this is the merge of partial softmax results given
 * for ca_chunk_attention_split, applied only where it pays.  One launch of one
 * workgroup per compute unit ("slot"); each derives the same plan from len:
 *   - a tile (32-row query blocks of 8 waves) has w work units, its table
 *     entries up to the last block its rows may see; A = the even share of
 *     the total per slot, at least 32; a job costs about 12 units on its own;
 *   - when the longest walk is within 24 units of A nothing is cut (slot s
 *     runs tile s); otherwise slot s runs tile s, whole when w - A <
 *     max(A/8, 24), else its first A units, then its share of the cut tiles'
 *     remaining units, laid end to end (filling each slot to A less one job
 *     cost);
 *   - a tile run whole writes O and lse; the pieces of a cut tile write
 *     partial results to the workspace, and a second kernel merges them (as
 *     in ca_chunk_attention_split).
 * Same result as ca_chunk_attention (the same admissible keys and softmax),
 * bit for bit where nothing is cut, else up to the rounding of the merge.
 * Shapes with more tiles (B * H_kv * ceil(H_q/H_kv * ceil(C_max/32) / 8)) than
 * the device's compute units (or than 1024), or with tiles * NKB_max above
 * 2^31 - 1, run ca_chunk_attention.
 *
 * workspace  device memory owned by the caller, 16-byte aligned, at least
 *            ca_chunk_attention_balanced_workspace_size(B, H_q, H_kv, C_max, D)
 *            bytes (else CA_ERR_SHAPE; NULL gives CA_ERR_NULL).  Its contents
 *            need no initialisation (every call writes what it reads).  Calls
 *            that share one workspace must be ordered on one stream.
 * dtype      CA_BF16; CA_F32 runs ca_chunk_attention (workspace unused).
 * Other arguments, layouts and errors as for ca_chunk_attention.
 */
CA_EXPORT ca_status ca_chunk_attention_balanced(const void* Q, const void* K_cache,
                                      const void* V_cache, const int32_t* T, const int32_t* len,
                                      int NKB_max, const int32_t* prior_len,
                                      const int32_t* chunk_len, int B, int H_q, int H_kv,
                                      int C_max, int64_t L, int D, int block, float scale,
                                      ca_dtype dtype, void* workspace, size_t workspace_bytes,
                                      void* O, float* lse, hipStream_t stream);

/* Bytes of workspace ca_chunk_attention_balanced needs, with tiles as above
 * and parts = 2 * tiles + 1024 (the most partial tiles a call on up to 1024
 * compute units writes): parts * 256 * (D + 2) * 4 bytes of partial results
 * and (tiles + 1) * 4 bytes of part numbering (each part 16-byte aligned); 16
 * for shapes with more than 1024 tiles (they run ca_chunk_attention); 0 for
 * invalid sizes (H_q % H_kv != 0, D not 64 or 128, nonpositive sizes). */
CA_EXPORT size_t ca_chunk_attention_balanced_workspace_size(int B, int H_q, int H_kv,
                                                            int C_max, int D);

/*
 * ca_chunk_attention_rows -- the block-sparse-kernel execution that the union
 * replaces: each 64-row Q-block of each query head attends its own mask row,
 * with no union over Q-blocks or heads.  CompactAttention, abstract and
 * "Methodology": block-sparse kernels take the 2D mask as the execution plan,
 * which loses efficiency when a chunk bounds the number of queries per KV
 * list; the union turns the mask into selection signals instead.  A baseline
 * for measurement beside ca_chunk_attention.
 *
 * Same as ca_chunk_attention, except that for chunk row i of head h
 *
 *   A = { t : T_rows[b,h,i/64,j] == t/64 for some j < len_rows[b,h,i/64],  t <= p }
 *
 * T_rows      device int32 [B, H_q, NQ_max, NKB_max], each row strictly
 *             ascending then -1 (see ca_build_union_tables for how to build it).
 * len_rows    device int32 [B, H_q, NQ_max].
 * NQ_max      Q-blocks per head in T_rows; 64 * NQ_max >= C_max (else CA_ERR_SHAPE).
 * Other arguments, layouts and errors as for ca_chunk_attention.  A workgroup
 * of the bf16 path holds one Q-block of one head (64 query rows per KV tile
 * staged, against up to 256 in ca_chunk_attention).
 */
CA_EXPORT ca_status ca_chunk_attention_rows(const void* Q, const void* K_cache,
                                  const void* V_cache, const int32_t* T_rows,
                                  const int32_t* len_rows, int NQ_max, int NKB_max,
                                  const int32_t* prior_len, const int32_t* chunk_len, int B,
                                  int H_q, int H_kv, int C_max, int64_t L, int D, int block,
                                  float scale, ca_dtype dtype, void* O, float* lse,
                                  hipStream_t stream);

/*
 * ca_check_tables -- checks tables against the contract that
 * ca_chunk_attention relies on without checking it on the device (selection
 * stage output: minimal tables, strictly ascending, padded).  For each
 * pseudo-request u = b*H_kv + g, row_bad[u] is a bitmask, 0 when the row is
 * well formed:
 *   1  len[u] outside [0, NKB_max]
 *   2  an entry T[b,g,j], j < len[u], outside [0, n_kv_blocks[b])
 *   4  T[b,g,0 .. len[u]) not strictly ascending (a repeat counts)
 *   8  an entry past len[u] (padding) other than -1
 * (with len[u] out of range, entries are judged against len clamped to
 * [0, NKB_max]).  Tables from ca_build_union_tables give all zeros.
 * T, len       device int32 [B, H_kv, NKB_max] and [B, H_kv].
 * n_kv_blocks  host int32 [B], each in [0, NKB_max] (else CA_ERR_SHAPE).
 * row_bad      device int32 [B * H_kv] (out), owned by the caller.
 * Asynchronous on `stream`; a caller who wants the answer on the host copies
 * row_bad back.  Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_HIP.
 */
CA_EXPORT ca_status ca_check_tables(const int32_t* T, const int32_t* len, int B, int H_kv,
                                    int NKB_max, const int32_t* n_kv_blocks, int32_t* row_bad,
                                    hipStream_t stream);

/*
 * ca_tables_to_csr -- the paged-metadata view of the tables (execution stage:
 * the tables travel to a paged dense kernel as kv_indptr / kv_indices).
 * Pseudo-request u = b*H_kv + g.
 *
 *   kv_indptr[0] = 0, kv_indptr[u+1] = kv_indptr[u] + len[u]
 *   kv_indices[kv_indptr[u] + j] = u * (L/64) + T[b,g,j]      (j < len[u])
 *
 * i.e. global page ids of the cache viewed as [B*H_kv*L/64, 64, D].
 * T, len      device, as produced by ca_build_union_tables (len in [0, NKB_max]).
 * L           cache capacity in tokens; a multiple of 64 (else CA_ERR_SHAPE).
 * kv_indptr   device int32 [B*H_kv + 1] (out).
 * kv_indices  device int32 with room for B*H_kv*NKB_max entries (out; only the
 *             first kv_indptr[B*H_kv] are written).
 * Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_HIP.
 */
CA_EXPORT ca_status ca_tables_to_csr(const int32_t* T, const int32_t* len, int B, int H_kv, int NKB_max,
                           int64_t L, int32_t* kv_indptr, int32_t* kv_indices,
                           hipStream_t stream);

/*
 * ca_append_kv -- the append step of chunked prefill (problem statement of
 * the technical summaries: chunks are processed in sequence, and each attends
 * to the cache accumulated so far plus itself, so its own keys and values are
 * written into the cache before ca_chunk_attention runs).
 *
 *   K_cache[b, g, prior_len[b] + i, :] = K_new[b, g, i, :]   (i < chunk_len[b]),
 *   V_cache likewise; every other cache row is left as it was.
 *
 * K_new, V_new      device [B, H_kv, C_max, D] (dtype), 16-byte aligned: the
 *                   chunk's keys and values, rows [0, chunk_len[b]) used.
 * K_cache, V_cache  device [B, H_kv, L, D] (dtype), 16-byte aligned (in/out).
 * prior_len, chunk_len  host int32 [B]; 0 <= chunk_len[b] <= C_max,
 *                   prior_len[b] >= 0, prior_len[b] + chunk_len[b] <= L (else
 *                   CA_ERR_SHAPE).  Any row offsets (no multiple of 64 needed).
 * B in [1, CA_MAX_BATCH], B*H_kv <= 2^24, D in {64, 128}.  The new rows must
 * not overlap the cache.  Asynchronous on `stream`.
 * Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_DTYPE, CA_ERR_UNSUPPORTED, CA_ERR_HIP.
 */
CA_EXPORT ca_status ca_append_kv(const void* K_new, const void* V_new, int B, int H_kv, int C_max,
                                 int64_t L, int D, ca_dtype dtype, const int32_t* prior_len,
                                 const int32_t* chunk_len, void* K_cache, void* V_cache,
                                 hipStream_t stream);

/*
 * ca_compact_kv -- explicit KV compaction: the selected blocks are gathered
 * into a compact buffer before a dense kernel runs.  CompactAttention,
 * abstract: its block tables let the attention read the selected blocks in
 * place, so this copy (the KV-copy overhead it names for token-level
 * selection) is avoided.  A baseline to measure that saving against, not part
 * of the zero-copy path.
 *
 * For each (b, g) with n = len[b,g] entries, of which the first p are prior
 * blocks (T[b,g,j] < prior_len[b]/64), block T[b,g,j] of K_cache/V_cache is
 * copied to block
 *     dst(j) = prior_len[b]/64 - p + j   (j < p: prior blocks, packed to end
 *                                         where the chunk starts)
 *     dst(j) = T[b,g,j]                 (j >= p: current-chunk blocks stay)
 * of K_out/V_out, and T_out[b,g,j] = dst(j) (then -1 up to NKB_max).  So
 * ca_chunk_attention(Q, K_out, V_out, T_out, len, prior_len, chunk_len, ...)
 * computes exactly what it computes on the original cache and table (same
 * blocks, same order, same causal positions).  Entries outside
 * [0, (prior_len+chunk_len)/64), or whose destination would fall outside it,
 * are not copied and get T_out = -1.
 *
 * K_cache, V_cache  device [B, H_kv, L, D] (dtype), 16-byte aligned.
 * T, len            device, as produced by ca_build_union_tables (ascending).
 * K_out, V_out      device [B, H_kv, L, D] (out); blocks not selected are not written.
 * T_out             device int32 [B, H_kv, NKB_max] (out).
 * prior_len, chunk_len  host int32 [B], as for ca_chunk_attention (multiples
 *                   of 64, prior+chunk <= min(L, 64*NKB_max)).
 * B in [1, CA_MAX_BATCH], B*H_kv <= 2^24, D in {64, 128}.
 * The outputs must not overlap the inputs.  Asynchronous on `stream`.
 * Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_DTYPE, CA_ERR_UNSUPPORTED, CA_ERR_HIP.
 */
CA_EXPORT ca_status ca_compact_kv(const void* K_cache, const void* V_cache, const int32_t* T,
                                  const int32_t* len, int NKB_max, const int32_t* prior_len,
                                  const int32_t* chunk_len, int B, int H_kv, int64_t L, int D,
                                  ca_dtype dtype, void* K_out, void* V_out, int32_t* T_out,
                                  hipStream_t stream);

/*
 * Block-mask producer -- the step upstream of the union.  CompactAttention,
 * "Methodology" (selection stage) and the problem statement of the technical
 * summaries: the union consumes a per-head 2D block mask made by a
 * lightweight pattern search, which runs again over the growing KV cache at
 * every chunk.  The pages leave the searcher open; this one is training-free:
 * mean-pooled Q-block . mean-pooled KV-block scores, then per-row top-k.
 *
 * ca_pool_blocks -- out[b,h,kb,:] = mean over r < 64 of X[b,h,64*kb + r,:]
 * for blk_begin[b] <= kb < blk_end[b]; every other entry of `out` is left as
 * it was (so pooled keys can be kept across chunks and only new blocks pooled).
 *   X           device [B, H, R, D], element type `dtype` (bf16 or fp32),
 *               16-byte aligned.
 *   blk_begin,  host int32 [B]; 0 <= blk_begin[b] <= blk_end[b] <= NB_out,
 *   blk_end     64 * blk_end[b] <= R, blk_end[b] - blk_begin[b] <= 65535.
 *   out         device float [B, H, NB_out, D], 16-byte aligned.
 *   B in [1, CA_MAX_BATCH], B*H <= 2^24, D in {64, 128}.
 *   Sums are fp32, in a fixed order.
 * Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_DTYPE, CA_ERR_UNSUPPORTED, CA_ERR_HIP.
 */
CA_EXPORT ca_status ca_pool_blocks(const void* X, ca_dtype dtype, int B, int H, int64_t R, int D,
                         const int32_t* blk_begin, const int32_t* blk_end, float* out,
                         int NB_out, hipStream_t stream);

/*
 * ca_block_mask_topk -- block scores and the mask built from them.  With
 * P = prior_len[b]/64, nq = chunk_len[b]/64, g = h / (H_q/H_kv):
 *
 *   scores[b,h,qb,kb] = sum_d qbar[b,h,qb,d] * kbar[b,g,kb,d]  (qb < nq, kb < P;
 *                       each fp32 value split into bf16 hi + lo parts, the
 *                       products hi*hi + hi*lo + lo*hi summed in fp32 on the
 *                       bf16 matrix cores: within 3 * 2^-16 sum_d |q_d k_d|
 *                       of the fp32 dot product, plus fp32 accumulation)
 *   mask[b,h,qb,kb]   = 1 for kb = 0 (when P > 0), for P - local <= kb < P,
 *                       for P <= kb <= P + qb (causal block triangle), and for
 *                       the `budget` candidates 1 <= kb < max(P - local, 1)
 *                       with the highest scores (ties: lower kb first; all of
 *                       them when there are fewer); 0 elsewhere and on every
 *                       row qb >= nq.
 *
 *   qbar        device float [B, H_q, NQ_max, D] (pooled Q-blocks), 16-byte aligned.
 *   kbar        device float [B, H_kv, NKB_max, D] (pooled KV blocks; rows
 *               kb < P must be valid), 16-byte aligned.
 *   prior_len,  host int32 [B], multiples of 64 (else CA_ERR_UNSUPPORTED);
 *   chunk_len   chunk_len <= 64*NQ_max, prior_len + chunk_len <= 64*NKB_max.
 *   budget, local  >= 0.
 *   scores      device float [B, H_q, NQ_max, NKB_max] (out; entries with
 *               qb >= nq or kb >= P are not written).  Scratch owned by the caller.
 *   mask        device uint8 [B, H_q, NQ_max, NKB_max] (out, fully written): the
 *               input of ca_build_union_tables.
 *   B*H_kv <= 65535, D in {64, 128}.
 * Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_UNSUPPORTED, CA_ERR_HIP.
 */
CA_EXPORT ca_status ca_block_mask_topk(const float* qbar, const float* kbar, int B, int H_q,
                             int H_kv, int NQ_max, int NKB_max, int D,
                             const int32_t* prior_len, const int32_t* chunk_len, int budget,
                             int local, float* scores, uint8_t* mask, hipStream_t stream);

/*
 * ca_select_chunk -- the whole selection step of one chunk in four launches
 * (problem statement and "Methodology", selection stage: the search runs over
 * the grown cache at every chunk, and its mask becomes the union tables).
 * Same outputs as the calls it fuses, bit for bit:
 *
 *   ca_pool_blocks(K_cache -> kbar, blocks [prior/64, (prior+chunk)/64))
 *   ca_pool_blocks(Q_chunk -> qbar, blocks [0, chunk/64))
 *   ca_block_mask_topk(qbar, kbar, prior, chunk, budget, local -> scores, mask)
 *   ca_build_union_tables(mask, n_q_blocks = chunk/64,
 *                         n_kv_blocks = (prior+chunk)/64 -> T, len)
 *
 * The launches: pooling of the new key blocks and of the Q-blocks together
 * (which also clears the union bitmap words kept at the tail of each T row),
 * the scores, the top-k mask with each selected cell ORed into its group's
 * bitmap, and the compaction of the bitmaps into T and len.  The mask is read
 * by nothing: the union comes from the selection directly.
 *
 * Q_chunk    device [B, H_q, C_max, D] (dtype), 16-byte aligned.
 * K_cache    device [B, H_kv, L, D] (dtype), 16-byte aligned; rows up to
 *            prior_len[b] + chunk_len[b] hold the keys (append first).
 * prior_len, chunk_len  host int32 [B], multiples of 64 (else
 *            CA_ERR_UNSUPPORTED); chunk_len <= min(C_max, 64*NQ_max),
 *            prior_len + chunk_len <= min(L, 64*NKB_max).
 * qbar       device float [B, H_q, NQ_max, D] (out; the chunk's Q-blocks).
 * kbar       device float [B, H_kv, NKB_max, D] (in/out: blocks below
 *            prior/64 must hold the pooled keys of earlier chunks; the
 *            chunk's own blocks are written).  16-byte aligned.
 * scores, mask  as for ca_block_mask_topk.
 * T, len     as for ca_build_union_tables (NKB_max <= 524288).
 * B*H_kv <= 65535, D in {64, 128}, budget, local >= 0.
 * Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_DTYPE, CA_ERR_UNSUPPORTED, CA_ERR_HIP.
 */
CA_EXPORT ca_status ca_select_chunk(const void* Q_chunk, const void* K_cache, ca_dtype dtype,
                                    int B, int H_q, int H_kv, int C_max, int64_t L, int D,
                                    const int32_t* prior_len, const int32_t* chunk_len,
                                    int budget, int local, float* qbar, int NQ_max, float* kbar,
                                    int NKB_max, float* scores, uint8_t* mask, int32_t* T,
                                    int32_t* len, hipStream_t stream);

/*
 * ca_append_select_chunk -- a chunk's append (ca_append_kv) and its selection
 * (ca_select_chunk) in the four launches of the selection: the first launch
 * also copies the chunk's keys and values into the caches, and pools the new
 * key blocks from the rows it copies instead of reading them back from the
 * cache (problem statement of the technical summaries: each chunk's K/V join
 * the cache before it attends, and the search runs again over the grown
 * cache).  Outputs are those of
 *
 *   ca_append_kv(K_new, V_new, ..., prior_len, chunk_len, K_cache, V_cache)
 *   ca_select_chunk(Q_chunk, K_cache, ..., prior_len, chunk_len, ...)
 *
 * bit for bit (caches, kbar, qbar, scores, mask, T, len).
 *
 * K_new, V_new  device [B, H_kv, C_max, D] (dtype), 16-byte aligned: the
 *               chunk's keys and values, rows [0, chunk_len[b]) used.
 * K_cache, V_cache  device [B, H_kv, L, D] (dtype), 16-byte aligned (in/out):
 *               rows [prior_len[b], prior_len[b] + chunk_len[b]) are written,
 *               rows below prior_len[b] must hold the earlier chunks.
 * Every other argument as for ca_select_chunk (prior_len and chunk_len
 * multiples of 64).  The new rows must not overlap the caches.
 * Errors: CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_DTYPE, CA_ERR_UNSUPPORTED, CA_ERR_HIP.
 */
CA_EXPORT ca_status ca_append_select_chunk(const void* K_new, const void* V_new,
                                           const void* Q_chunk, void* K_cache, void* V_cache,
                                           ca_dtype dtype, int B, int H_q, int H_kv, int C_max,
                                           int64_t L, int D, const int32_t* prior_len,
                                           const int32_t* chunk_len, int budget, int local,
                                           float* qbar, int NQ_max, float* kbar, int NKB_max,
                                           float* scores, uint8_t* mask, int32_t* T,
                                           int32_t* len, hipStream_t stream);

/*
 * ca_select_chunk_devlen, ca_append_select_chunk_devlen -- ca_select_chunk and
 * ca_append_select_chunk with prior_len and chunk_len in device memory
 * (problem statement of the technical summaries: the selection runs again for
 * every chunk as the cache grows; with the lengths in device memory, one
 * captured HIP graph of a chunk's selection, or of its whole step with
 * ca_chunk_attention_devlen, serves every chunk offset: between replays only
 * the device lengths and the inputs' contents change).
 *
 * prior_len,  device int32 [B], 4-byte aligned (else CA_ERR_UNSUPPORTED),
 * chunk_len   read by the kernels when they run and checked there: lengths
 *             that are negative, not multiples of 64, a chunk past
 *             min(C_max, 64*NQ_max) or a total past min(L, 64*NKB_max) make
 *             that sequence an empty chunk (nothing appended, pooled or
 *             selected; its mask rows 0 and its tables empty).
 * The grids are sized for the largest lengths those bounds allow.  With valid
 * lengths the outputs equal those of the host-length calls bit for bit.
 * Every other argument and the errors as for ca_select_chunk and
 * ca_append_select_chunk.
 */
CA_EXPORT ca_status ca_select_chunk_devlen(const void* Q_chunk, const void* K_cache,
                                           ca_dtype dtype, int B, int H_q, int H_kv, int C_max,
                                           int64_t L, int D, const int32_t* prior_len,
                                           const int32_t* chunk_len, int budget, int local,
                                           float* qbar, int NQ_max, float* kbar, int NKB_max,
                                           float* scores, uint8_t* mask, int32_t* T,
                                           int32_t* len, hipStream_t stream);
CA_EXPORT ca_status ca_append_select_chunk_devlen(
    const void* K_new, const void* V_new, const void* Q_chunk, void* K_cache, void* V_cache,
    ca_dtype dtype, int B, int H_q, int H_kv, int C_max, int64_t L, int D,
    const int32_t* prior_len, const int32_t* chunk_len, int budget, int local, float* qbar,
    int NQ_max, float* kbar, int NKB_max, float* scores, uint8_t* mask, int32_t* T, int32_t* len,
    hipStream_t stream);

/* Human-readable name of a status code (static string; never NULL). */
CA_EXPORT const char* ca_status_string(ca_status s);

/* Text of the last HIP error seen by a call on this thread ("" if none). */
CA_EXPORT const char* ca_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* COMPACT_ATTN_H */
