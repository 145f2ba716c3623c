// C ABI of the CompactAttention chunked-prefill path: host-side validation,
// scheduling metadata and kernel launches.  The library allocates nothing and
// keeps no state beyond a per-thread copy of the last HIP error text and a
// per-device cache of the compute-unit count (the static scratch array of
// ca_chunk_attention_split_noalloc lives in static_scratch.hip).

#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <numeric>

#include "kernels.hpp"

namespace {

thread_local char g_last_hip_error[256] = "";

ca_status hip_status(hipError_t e) {
  if (e == hipSuccess) return CA_OK;
  snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s (%d)", hipGetErrorString(e),
           static_cast<int>(e));
  return CA_ERR_HIP;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

constexpr int kMaxUnionBlocks = 1 << 19;  // NKB_max bound: bitmap fits 64 KiB of LDS
constexpr int kCUs = 256;                 // compute units of a whole MI355X

// Compute units of the current device, queried once per device (a
// partitioned MI355X exposes fewer); the full chip's count if the query fails.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kCUs;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = kCUs;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

extern "C" {

CA_EXPORT const char* ca_status_string(ca_status s) {
  switch (s) {
    case CA_OK: return "CA_OK";
    case CA_ERR_NULL: return "CA_ERR_NULL: a required pointer is NULL";
    case CA_ERR_SHAPE: return "CA_ERR_SHAPE: sizes inconsistent or out of range";
    case CA_ERR_DTYPE: return "CA_ERR_DTYPE: unknown element type";
    case CA_ERR_UNSUPPORTED: return "CA_ERR_UNSUPPORTED: request this library does not run";
    case CA_ERR_HIP: return "CA_ERR_HIP: the HIP runtime reported an error";
    case CA_ERR_TOO_LARGE:
      return "CA_ERR_TOO_LARGE: the call needs more than the library's static scratch memory";
  }
  return "unknown ca_status";
}

CA_EXPORT const char* ca_last_hip_error(void) { return g_last_hip_error; }

CA_EXPORT ca_status ca_build_union_tables(const uint8_t* mask, int B, int H_q, int H_kv,
                                          int NQ_max, int NKB_max, const int32_t* n_q_blocks,
                                          const int32_t* n_kv_blocks, int32_t* T, int32_t* len,
                                          hipStream_t stream) {
  if (!mask || !n_q_blocks || !n_kv_blocks || !T || !len) return CA_ERR_NULL;
  if (B < 1 || B > CA_MAX_BATCH || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || NQ_max < 1 ||
      NKB_max < 1 || NKB_max > kMaxUnionBlocks)
    return CA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H_kv > (1 << 30)) return CA_ERR_SHAPE;
  ca::UnionExtents ext;
  memset(&ext, 0, sizeof(ext));
  for (int b = 0; b < B; ++b) {
    if (n_q_blocks[b] < 0 || n_q_blocks[b] > NQ_max || n_kv_blocks[b] < 0 ||
        n_kv_blocks[b] > NKB_max)
      return CA_ERR_SHAPE;
    ext.nq[b] = n_q_blocks[b];
    ext.nkb[b] = n_kv_blocks[b];
  }
  return hip_status(ca::launch_union_tables(mask, B, H_q, H_kv, NQ_max, NKB_max, ext, nullptr,
                                            nullptr, T, len, device_cus(), stream));
}

CA_EXPORT ca_status ca_build_union_tables_devlen(const uint8_t* mask, int B, int H_q, int H_kv,
                                                 int NQ_max, int NKB_max,
                                                 const int32_t* n_q_blocks,
                                                 const int32_t* n_kv_blocks, int32_t* T,
                                                 int32_t* len, hipStream_t stream) {
  if (!mask || !n_q_blocks || !n_kv_blocks || !T || !len) return CA_ERR_NULL;
  if (B < 1 || B > CA_MAX_BATCH || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || NQ_max < 1 ||
      NKB_max < 1 || NKB_max > kMaxUnionBlocks)
    return CA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H_kv > (1 << 30)) return CA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(n_q_blocks) | reinterpret_cast<uintptr_t>(n_kv_blocks)) & 3u)
    return CA_ERR_UNSUPPORTED;
  ca::UnionExtents ext;  // unused: the kernel reads the extents from device memory
  memset(&ext, 0, sizeof(ext));
  return hip_status(ca::launch_union_tables(mask, B, H_q, H_kv, NQ_max, NKB_max, ext,
                                            n_q_blocks, n_kv_blocks, T, len, device_cus(),
                                            stream));
}

CA_EXPORT ca_status ca_check_tables(const int32_t* T, const int32_t* len, int B, int H_kv,
                                    int NKB_max, const int32_t* n_kv_blocks, int32_t* row_bad,
                                    hipStream_t stream) {
  if (!T || !len || !n_kv_blocks || !row_bad) return CA_ERR_NULL;
  if (B < 1 || B > CA_MAX_BATCH || H_kv < 1 || NKB_max < 1) return CA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H_kv > (1 << 30)) return CA_ERR_SHAPE;
  ca::UnionExtents ext;
  memset(&ext, 0, sizeof(ext));
  for (int b = 0; b < B; ++b) {
    if (n_kv_blocks[b] < 0 || n_kv_blocks[b] > NKB_max) return CA_ERR_SHAPE;
    ext.nkb[b] = n_kv_blocks[b];
  }
  return hip_status(ca::launch_check_tables(T, len, B * H_kv, H_kv, NKB_max, ext, row_bad,
                                            stream));
}

CA_EXPORT ca_status ca_tables_to_csr(const int32_t* T, const int32_t* len, int B, int H_kv,
                                     int NKB_max, int64_t L, int32_t* kv_indptr,
                                     int32_t* kv_indices, hipStream_t stream) {
  if (!T || !len || !kv_indptr || !kv_indices) return CA_ERR_NULL;
  if (B < 1 || B > CA_MAX_BATCH || H_kv < 1 || NKB_max < 1 || L < CA_BLOCK || L % CA_BLOCK != 0)
    return CA_ERR_SHAPE;
  const int64_t pages = L / CA_BLOCK;
  const int64_t n_bg = static_cast<int64_t>(B) * H_kv;
  // page ids and entry counts must fit int32
  if (n_bg * pages > INT32_MAX || n_bg * NKB_max > INT32_MAX || NKB_max > pages)
    return CA_ERR_SHAPE;
  return hip_status(ca::launch_tables_to_csr(T, len, static_cast<int>(n_bg), NKB_max, pages,
                                             kv_indptr, kv_indices, stream));
}

}  // extern "C"

namespace {

// Byte offsets of the balanced path's workspace parts (each 16-byte aligned)
// and its total size.  A part is one cut tile's partial results (256 rows of D
// floats, then 256 (max, denominator) pairs); a call with n tiles on up to
// kPlanMaxSlots slots writes at most 2 n + kPlanMaxSlots parts; then the
// plan's part numbering (n + 1 ints).  Shapes with more tiles than
// kPlanMaxSlots always run the plain kernel and use no workspace.
struct BalancedLayout {
  size_t part_o, part_ml, pre, total;
  int64_t units, parts;
};
BalancedLayout balanced_layout(int B, int H_q, int H_kv, int C_max, int D) {
  auto up16 = [](size_t x) { return (x + 15) & ~static_cast<size_t>(15); };
  const int64_t n_pb = (static_cast<int64_t>(C_max) + 31) / 32;
  BalancedLayout l;
  l.units = static_cast<int64_t>(B) * H_kv * (((H_q / H_kv) * n_pb + 7) / 8);
  l.part_o = l.part_ml = l.pre = 0;
  if (l.units > ca::kPlanMaxSlots) {
    l.parts = 0;
    l.total = 16;
    return l;
  }
  l.parts = 2 * l.units + ca::kPlanMaxSlots;
  const size_t rows = static_cast<size_t>(l.parts) * 256;
  l.part_ml = up16(rows * D * sizeof(float));
  l.pre = up16(l.part_ml + rows * 2 * sizeof(float));
  l.total = up16(l.pre + static_cast<size_t>(l.units + 1) * sizeof(int32_t));
  return l;
}

// Shared by both table layouts: validation, sequence order, launch parameters.
ca_status attention(const void* Q, const void* K_cache, const void* V_cache, const int32_t* T,
                    const int32_t* len, int NQ_max, int NKB_max, const int32_t* prior_len,
                    const int32_t* chunk_len, int B, int H_q, int H_kv, int C_max, int64_t L,
                    int D, int block, float scale, ca_dtype dtype, void* O, float* lse,
                    bool row_tables, int n_split, void* workspace, size_t workspace_bytes,
                    hipStream_t stream, bool balanced = false, bool static_scratch = false,
                    bool dev_lengths = false, uint32_t* stamps = nullptr,
                    int max_stamped = 0, int* n_stamped = nullptr) {
  if (!Q || !K_cache || !V_cache || !T || !len || !prior_len || !chunk_len || !O)
    return CA_ERR_NULL;
  if (dtype != CA_F32 && dtype != CA_BF16) return CA_ERR_DTYPE;
  if (B < 1 || B > CA_MAX_BATCH || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || C_max < 1 ||
      L < 1 || NKB_max < 1 || !(scale > 0.f) || !isfinite(scale))
    return CA_ERR_SHAPE;
  if (row_tables && NQ_max * CA_BLOCK < C_max) return CA_ERR_SHAPE;
  if (block != CA_BLOCK || (D != 64 && D != 128)) return CA_ERR_UNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K_cache) || !aligned16(V_cache) || !aligned16(O) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return CA_ERR_UNSUPPORTED;
  ca::SeqInfo seq;
  memset(&seq, 0, sizeof(seq));
  if (dev_lengths) {
    // lengths stay on the device (the kernels check them); sequences in order
    if ((reinterpret_cast<uintptr_t>(prior_len) | reinterpret_cast<uintptr_t>(chunk_len)) & 3u)
      return CA_ERR_UNSUPPORTED;
    for (int r = 0; r < B; ++r) seq.order[r] = r;
  } else {
    int64_t work[CA_MAX_BATCH];
    for (int b = 0; b < B; ++b) {
      const int64_t P = prior_len[b], C = chunk_len[b];
      if (P < 0 || C < 0 || C > C_max || P + C > L ||
          P + C > static_cast<int64_t>(NKB_max) * CA_BLOCK)
        return CA_ERR_SHAPE;
      if (P % CA_BLOCK != 0 || C % CA_BLOCK != 0) return CA_ERR_UNSUPPORTED;
      seq.prior[b] = static_cast<int32_t>(P);
      seq.chunk[b] = static_cast<int32_t>(C);
      work[b] = (P + C) * C;  // dense upper bound of the sequence's attention work
    }
    int order[CA_MAX_BATCH];
    std::iota(order, order + B, 0);
    std::stable_sort(order, order + B, [&](int a, int c) { return work[a] > work[c]; });
    for (int r = 0; r < B; ++r) seq.order[r] = order[r];
  }

  ca::AttnParams p;
  p.H_q = H_q;
  p.H_kv = H_kv;
  p.G = H_q / H_kv;
  p.C_max = C_max;
  p.L = L;
  p.NKB_max = NKB_max;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.waves = 4;
  p.row_tables = row_tables ? 1 : 0;
  p.NQ_max = row_tables ? NQ_max : 0;
  p.n_split = n_split;
  p.rows_total = static_cast<int64_t>(B) * H_q * C_max;
  p.cus = device_cus();
  p.bal_units = 0;
  p.bal_parts = 0;
  p.bal_pre = nullptr;
  p.dev_prior = dev_lengths ? prior_len : nullptr;
  p.dev_chunk = dev_lengths ? chunk_len : nullptr;
  p.stamps = nullptr;
  const int64_t n_bg = static_cast<int64_t>(B) * H_kv;
  if (dtype == CA_BF16) {
    // the bf16 kernels address one (b, g) cache slice through a buffer
    // resource with 32-bit byte offsets
    if (L * D * 2 > static_cast<int64_t>(UINT32_MAX)) return CA_ERR_UNSUPPORTED;
    const int64_t n_pb = (C_max + 31) / 32;
    // workgroups per (b, g): 8 waves of 32 rows over the group's heads while
    // that still gives every CU a workgroup, else 4 (and 4 with split-KV); or
    // one 64-row Q-block of one head with per-Q-block tables
    const int64_t n_t8 = (p.G * n_pb + 7) / 8;
    if (balanced) {
      // planned in the kernel while every tile has a slot (one workgroup per
      // compute unit) and the plan's sums fit in 32 bits; otherwise the plain
      // kernel below, which gives the same result
      const BalancedLayout ws = balanced_layout(B, H_q, H_kv, C_max, D);
      const int64_t units = n_bg * n_t8;
      const int slots = std::min(p.cus, ca::kPlanMaxSlots);
      if (units <= slots && units * NKB_max <= INT32_MAX) {
        p.waves = 8;
        p.n_t = static_cast<int>(n_t8);
        p.xcd = (n_bg % 8 == 0) ? 1 : 0;
        p.bal_units = static_cast<int>(units);
        p.bal_parts = static_cast<int>(ws.parts);
        char* base = static_cast<char*>(workspace);
        float* part_o = reinterpret_cast<float*>(base + ws.part_o);
        float* part_ml = reinterpret_cast<float*>(base + ws.part_ml);
        p.bal_pre = reinterpret_cast<int32_t*>(base + ws.pre);
        return hip_status(ca::launch_chunk_attn_bf16_balanced(Q, K_cache, V_cache, T, len, O,
                                                              lse, D, p, seq, part_o, part_ml,
                                                              slots, stream));
      }
    }
    p.waves = (n_split == 1 && n_bg * n_t8 >= p.cus) ? 8 : 4;
    p.n_t = row_tables ? static_cast<int>(p.G * ((C_max + 63) / 64))
                       : static_cast<int>((p.G * n_pb + p.waves - 1) / p.waves);
    p.xcd = (n_bg % 8 == 0) ? 1 : 0;
    if (n_bg * p.n_t * n_split > INT32_MAX) return CA_ERR_SHAPE;
    if (n_stamped != nullptr) {  // stamped call: one record per workgroup
      const int64_t n_wg = n_bg * p.n_t;
      *n_stamped = static_cast<int>(n_wg);
      if (n_wg > max_stamped) return CA_ERR_SHAPE;
      p.stamps = stamps;
    }
    if (n_split > 1) {
      if (static_scratch) {  // every argument checked: now look up the array
        hipError_t e = hipSuccess;
        workspace = ca::static_scratch_address(&e);
        if (workspace == nullptr) return hip_status(e);
      }
      float* part_o = static_cast<float*>(workspace);
      float* part_ml = part_o + static_cast<size_t>(n_split) * p.rows_total * D;
      return hip_status(ca::launch_chunk_attn_bf16_split(Q, K_cache, V_cache, T, len, O, lse, B,
                                                         D, p, seq, part_o, part_ml, stream));
    }
    return hip_status(ca::launch_chunk_attn_bf16(Q, K_cache, V_cache, T, len, O, lse, B, D, p,
                                                 seq, stream));
  }
  p.n_t = 0;
  p.xcd = 0;
  if (static_cast<int64_t>(B) * H_q * n_split * ((C_max + 31) / 32) > INT32_MAX)
    return CA_ERR_SHAPE;
  const float* q = static_cast<const float*>(Q);
  const float* k = static_cast<const float*>(K_cache);
  const float* v = static_cast<const float*>(V_cache);
  if (n_split > 1) {
    if (static_scratch) {
      hipError_t e = hipSuccess;
      workspace = ca::static_scratch_address(&e);
      if (workspace == nullptr) return hip_status(e);
    }
    float* part_o = static_cast<float*>(workspace);
    float* part_ml = part_o + static_cast<size_t>(n_split) * p.rows_total * D;
    return hip_status(ca::launch_chunk_attn_f32_split(q, k, v, T, len, static_cast<float*>(O),
                                                      lse, B, D, p, seq, part_o, part_ml,
                                                      stream));
  }
  return hip_status(
      ca::launch_chunk_attn_f32(q, k, v, T, len, static_cast<float*>(O), lse, B, D, p, seq,
                                stream));
}

}  // namespace

extern "C" {

CA_EXPORT ca_status ca_chunk_attention(const void* Q, const void* K_cache, const void* V_cache,
                                       const int32_t* T, const int32_t* len, int NKB_max,
                                       const int32_t* prior_len, const int32_t* chunk_len,
                                       int B, int H_q, int H_kv, int C_max, int64_t L, int D,
                                       int block, float scale, ca_dtype dtype, void* O,
                                       float* lse, hipStream_t stream) {
  return attention(Q, K_cache, V_cache, T, len, 0, NKB_max, prior_len, chunk_len, B, H_q, H_kv,
                   C_max, L, D, block, scale, dtype, O, lse, false, 1, nullptr, 0, stream);
}

CA_EXPORT ca_status ca_chunk_attention_devlen(const void* Q, const void* K_cache,
                                              const void* V_cache, const int32_t* T,
                                              const int32_t* len, int NKB_max,
                                              const int32_t* prior_len, const int32_t* chunk_len,
                                              int B, int H_q, int H_kv, int C_max, int64_t L,
                                              int D, int block, float scale, ca_dtype dtype,
                                              void* O, float* lse, hipStream_t stream) {
  return attention(Q, K_cache, V_cache, T, len, 0, NKB_max, prior_len, chunk_len, B, H_q, H_kv,
                   C_max, L, D, block, scale, dtype, O, lse, false, 1, nullptr, 0, stream, false,
                   false, true);
}

CA_EXPORT ca_status ca_chunk_attention_stamped(const void* Q, const void* K_cache,
                                               const void* V_cache, const int32_t* T,
                                               const int32_t* len, int NKB_max,
                                               const int32_t* prior_len,
                                               const int32_t* chunk_len, int B, int H_q,
                                               int H_kv, int C_max, int64_t L, int D, int block,
                                               float scale, ca_dtype dtype, void* O, float* lse,
                                               uint32_t* stamps, int max_workgroups,
                                               int* n_workgroups, hipStream_t stream) {
  if (!n_workgroups || (!stamps && max_workgroups > 0)) return CA_ERR_NULL;
  if (dtype != CA_BF16) return CA_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(stamps) & 3u) return CA_ERR_UNSUPPORTED;
  *n_workgroups = 0;
  return attention(Q, K_cache, V_cache, T, len, 0, NKB_max, prior_len, chunk_len, B, H_q, H_kv,
                   C_max, L, D, block, scale, dtype, O, lse, false, 1, nullptr, 0, stream, false,
                   false, false, stamps, max_workgroups, n_workgroups);
}

CA_EXPORT size_t ca_chunk_attention_workspace_size(int B, int H_q, int C_max, int D,
                                                    int n_splits) {
  if (B < 1 || H_q < 1 || C_max < 1 || D < 1 || n_splits < 2) return 0;
  return static_cast<size_t>(n_splits) * B * H_q * C_max * (D + 2) * sizeof(float);
}

CA_EXPORT ca_status ca_chunk_attention_split(const void* Q, const void* K_cache,
                                             const void* V_cache, const int32_t* T,
                                             const int32_t* len, int NKB_max,
                                             const int32_t* prior_len, const int32_t* chunk_len,
                                             int B, int H_q, int H_kv, int C_max, int64_t L,
                                             int D, int block, float scale, ca_dtype dtype,
                                             int n_splits, void* workspace,
                                             size_t workspace_bytes, void* O, float* lse,
                                             hipStream_t stream) {
  if (n_splits < 1 || n_splits > CA_MAX_SPLITS) return CA_ERR_SHAPE;
  if (n_splits == 1)
    return attention(Q, K_cache, V_cache, T, len, 0, NKB_max, prior_len, chunk_len, B, H_q,
                     H_kv, C_max, L, D, block, scale, dtype, O, lse, false, 1, nullptr, 0, stream);
  if (!workspace) return CA_ERR_NULL;
  if (!aligned16(workspace)) return CA_ERR_UNSUPPORTED;
  if (B >= 1 && H_q >= 1 && C_max >= 1 && (D == 64 || D == 128) &&
      workspace_bytes < ca_chunk_attention_workspace_size(B, H_q, C_max, D, n_splits))
    return CA_ERR_SHAPE;
  return attention(Q, K_cache, V_cache, T, len, 0, NKB_max, prior_len, chunk_len, B, H_q, H_kv,
                   C_max, L, D, block, scale, dtype, O, lse, false, n_splits, workspace,
                   workspace_bytes, stream);
}

CA_EXPORT ca_status ca_chunk_attention_split_noalloc(
    const void* Q, const void* K_cache, const void* V_cache, const int32_t* T,
    const int32_t* len, int NKB_max, const int32_t* prior_len, const int32_t* chunk_len, int B,
    int H_q, int H_kv, int C_max, int64_t L, int D, int block, float scale, ca_dtype dtype,
    int n_splits, void* O, float* lse, hipStream_t stream) {
  if (n_splits < 1 || n_splits > CA_MAX_SPLITS) return CA_ERR_SHAPE;
  if (n_splits == 1)
    return attention(Q, K_cache, V_cache, T, len, 0, NKB_max, prior_len, chunk_len, B, H_q,
                     H_kv, C_max, L, D, block, scale, dtype, O, lse, false, 1, nullptr, 0, stream);
  // the partials must fit the static array; checked before anything touches the device
  if (B >= 1 && H_q >= 1 && C_max >= 1 && (D == 64 || D == 128) &&
      ca_chunk_attention_workspace_size(B, H_q, C_max, D, n_splits) > CA_STATIC_SCRATCH_BYTES)
    return CA_ERR_TOO_LARGE;
  // every split writes its partials for every live row before the merge reads
  // them, so nothing in the array needs clearing between calls; the array's
  // address is looked up only once the arguments have passed every check
  return attention(Q, K_cache, V_cache, T, len, 0, NKB_max, prior_len, chunk_len, B, H_q, H_kv,
                   C_max, L, D, block, scale, dtype, O, lse, false, n_splits, nullptr,
                   CA_STATIC_SCRATCH_BYTES, stream, false, true);
}

CA_EXPORT size_t ca_chunk_attention_balanced_workspace_size(int B, int H_q, int H_kv, int C_max,
                                                             int D) {
  if (B < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || C_max < 1 || (D != 64 && D != 128))
    return 0;
  return balanced_layout(B, H_q, H_kv, C_max, D).total;
}

CA_EXPORT ca_status ca_chunk_attention_balanced(const void* Q, const void* K_cache,
                                                const void* V_cache, const int32_t* T,
                                                const int32_t* len, int NKB_max,
                                                const int32_t* prior_len,
                                                const int32_t* chunk_len, int B, int H_q,
                                                int H_kv, int C_max, int64_t L, int D, int block,
                                                float scale, ca_dtype dtype, void* workspace,
                                                size_t workspace_bytes, void* O, float* lse,
                                                hipStream_t stream) {
  if (dtype == CA_F32)  // the fp32 path runs unplanned: the workspace is not used
    return attention(Q, K_cache, V_cache, T, len, 0, NKB_max, prior_len, chunk_len, B, H_q,
                     H_kv, C_max, L, D, block, scale, dtype, O, lse, false, 1, nullptr, 0, stream);
  if (!workspace) return CA_ERR_NULL;
  if (!aligned16(workspace)) return CA_ERR_UNSUPPORTED;
  const size_t need = ca_chunk_attention_balanced_workspace_size(B, H_q, H_kv, C_max, D);
  if (need > 0 && workspace_bytes < need) return CA_ERR_SHAPE;
  return attention(Q, K_cache, V_cache, T, len, 0, NKB_max, prior_len, chunk_len, B, H_q, H_kv,
                   C_max, L, D, block, scale, dtype, O, lse, false, 1, workspace, workspace_bytes,
                   stream, true);
}

CA_EXPORT ca_status ca_chunk_attention_rows(const void* Q, const void* K_cache,
                                            const void* V_cache, const int32_t* T_rows,
                                            const int32_t* len_rows, int NQ_max, int NKB_max,
                                            const int32_t* prior_len, const int32_t* chunk_len,
                                            int B, int H_q, int H_kv, int C_max, int64_t L,
                                            int D, int block, float scale, ca_dtype dtype,
                                            void* O, float* lse, hipStream_t stream) {
  return attention(Q, K_cache, V_cache, T_rows, len_rows, NQ_max, NKB_max, prior_len, chunk_len,
                   B, H_q, H_kv, C_max, L, D, block, scale, dtype, O, lse, true, 1, nullptr, 0,
                   stream);
}

CA_EXPORT ca_status ca_append_kv(const void* K_new, const void* V_new, int B, int H_kv,
                                 int C_max, int64_t L, int D, ca_dtype dtype,
                                 const int32_t* prior_len, const int32_t* chunk_len,
                                 void* K_cache, void* V_cache, hipStream_t stream) {
  if (!K_new || !V_new || !prior_len || !chunk_len || !K_cache || !V_cache) return CA_ERR_NULL;
  if (dtype != CA_F32 && dtype != CA_BF16) return CA_ERR_DTYPE;
  if (B < 1 || B > CA_MAX_BATCH || H_kv < 1 || C_max < 1 || L < 1 ||
      static_cast<int64_t>(B) * H_kv > (1 << 24))
    return CA_ERR_SHAPE;
  if (D != 64 && D != 128) return CA_ERR_UNSUPPORTED;
  if (!aligned16(K_new) || !aligned16(V_new) || !aligned16(K_cache) || !aligned16(V_cache))
    return CA_ERR_UNSUPPORTED;
  ca::SeqInfo seq;
  memset(&seq, 0, sizeof(seq));
  for (int b = 0; b < B; ++b) {
    const int64_t P = prior_len[b], C = chunk_len[b];
    if (P < 0 || C < 0 || C > C_max || P + C > L) return CA_ERR_SHAPE;
    seq.prior[b] = static_cast<int32_t>(P);
    seq.chunk[b] = static_cast<int32_t>(C);
    seq.order[b] = b;
  }
  const int esz = dtype == CA_BF16 ? 2 : 4;
  return hip_status(ca::launch_append_kv(K_new, V_new, B, H_kv, C_max, L, D, esz, seq, K_cache,
                                         V_cache, stream));
}

CA_EXPORT ca_status ca_compact_kv(const void* K_cache, const void* V_cache, const int32_t* T,
                                  const int32_t* len, int NKB_max, const int32_t* prior_len,
                                  const int32_t* chunk_len, int B, int H_kv, int64_t L, int D,
                                  ca_dtype dtype, void* K_out, void* V_out, int32_t* T_out,
                                  hipStream_t stream) {
  if (!K_cache || !V_cache || !T || !len || !prior_len || !chunk_len || !K_out || !V_out ||
      !T_out)
    return CA_ERR_NULL;
  if (dtype != CA_F32 && dtype != CA_BF16) return CA_ERR_DTYPE;
  if (B < 1 || B > CA_MAX_BATCH || H_kv < 1 || L < 1 || NKB_max < 1 ||
      static_cast<int64_t>(B) * H_kv > (1 << 24))
    return CA_ERR_SHAPE;
  if (D != 64 && D != 128) return CA_ERR_UNSUPPORTED;
  if (!aligned16(K_cache) || !aligned16(V_cache) || !aligned16(K_out) || !aligned16(V_out))
    return CA_ERR_UNSUPPORTED;
  ca::SeqInfo seq;
  memset(&seq, 0, sizeof(seq));
  for (int b = 0; b < B; ++b) {
    const int64_t P = prior_len[b], C = chunk_len[b];
    if (P < 0 || C < 0 || P + C > L || P + C > static_cast<int64_t>(NKB_max) * CA_BLOCK)
      return CA_ERR_SHAPE;
    if (P % CA_BLOCK != 0 || C % CA_BLOCK != 0) return CA_ERR_UNSUPPORTED;
    seq.prior[b] = static_cast<int32_t>(P);
    seq.chunk[b] = static_cast<int32_t>(C);
  }
  const int esz = dtype == CA_BF16 ? 2 : 4;
  return hip_status(ca::launch_compact_kv(K_cache, V_cache, T, len, NKB_max, B, H_kv, L, D, esz,
                                          seq, K_out, V_out, T_out, stream));
}

CA_EXPORT ca_status ca_pool_blocks(const void* X, ca_dtype dtype, int B, int H, int64_t R, int D,
                                   const int32_t* blk_begin, const int32_t* blk_end, float* out,
                                   int NB_out, hipStream_t stream) {
  if (!X || !blk_begin || !blk_end || !out) return CA_ERR_NULL;
  if (dtype != CA_F32 && dtype != CA_BF16) return CA_ERR_DTYPE;
  if (B < 1 || B > CA_MAX_BATCH || H < 1 || R < 1 || NB_out < 1 ||
      static_cast<int64_t>(B) * H > (1 << 24))
    return CA_ERR_SHAPE;
  if (D != 64 && D != 128) return CA_ERR_UNSUPPORTED;
  if (!aligned16(X) || !aligned16(out)) return CA_ERR_UNSUPPORTED;
  ca::BlockRange rng;
  memset(&rng, 0, sizeof(rng));
  int max_span = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t lo = blk_begin[b], hi = blk_end[b];
    if (lo < 0 || hi < lo || hi > NB_out || hi * CA_BLOCK > R) return CA_ERR_SHAPE;
    rng.begin[b] = static_cast<int32_t>(lo);
    rng.end[b] = static_cast<int32_t>(hi);
    max_span = std::max(max_span, static_cast<int>(hi - lo));
  }
  if (max_span > 65535) return CA_ERR_SHAPE;
  return hip_status(ca::launch_pool_blocks(X, dtype == CA_BF16 ? 2 : 4, B, H, R, D, rng, max_span,
                                           out, NB_out, stream));
}

CA_EXPORT ca_status ca_block_mask_topk(const float* qbar, const float* kbar, int B, int H_q,
                                       int H_kv, int NQ_max, int NKB_max, int D,
                                       const int32_t* prior_len, const int32_t* chunk_len,
                                       int budget, int local, float* scores, uint8_t* mask,
                                       hipStream_t stream) {
  if (!qbar || !kbar || !prior_len || !chunk_len || !scores || !mask) return CA_ERR_NULL;
  if (B < 1 || B > CA_MAX_BATCH || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || NQ_max < 1 ||
      NKB_max < 1 || budget < 0 || local < 0)
    return CA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H_q * NQ_max > INT32_MAX ||
      static_cast<int64_t>(B) * H_kv > 65535)
    return CA_ERR_SHAPE;
  if (D != 64 && D != 128) return CA_ERR_UNSUPPORTED;
  if (!aligned16(qbar) || !aligned16(kbar)) return CA_ERR_UNSUPPORTED;
  ca::SeqInfo seq;
  memset(&seq, 0, sizeof(seq));
  int max_pblk = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t P = prior_len[b], C = chunk_len[b];
    if (P < 0 || C < 0 || C > static_cast<int64_t>(NQ_max) * CA_BLOCK ||
        P + C > static_cast<int64_t>(NKB_max) * CA_BLOCK)
      return CA_ERR_SHAPE;
    if (P % CA_BLOCK != 0 || C % CA_BLOCK != 0) return CA_ERR_UNSUPPORTED;
    seq.prior[b] = static_cast<int32_t>(P);
    seq.chunk[b] = static_cast<int32_t>(C);
    seq.order[b] = b;
    max_pblk = std::max(max_pblk, static_cast<int>(P / CA_BLOCK));
  }
  return hip_status(ca::launch_block_mask(qbar, kbar, B, H_q, H_kv, NQ_max, NKB_max, D, seq,
                                          max_pblk, budget, local, scores, mask, stream));
}

}  // extern "C"

namespace {

// ca_select_chunk, ca_append_select_chunk and their device-length forms:
// checks, then the launches (app: the chunk's new rows to append, or null;
// dev_lengths: prior_len and chunk_len are device int32 [B], checked by the
// kernels).
ca_status select_chunk_common(const void* Q_chunk, const void* K_cache, ca_dtype dtype, int B,
                              int H_q, int H_kv, int C_max, int64_t L, int D,
                              const int32_t* prior_len, const int32_t* chunk_len, int budget,
                              int local, float* qbar, int NQ_max, float* kbar, int NKB_max,
                              float* scores, uint8_t* mask, int32_t* T, int32_t* len,
                              const ca::AppendSrc* app, bool dev_lengths, hipStream_t stream) {
  if (!Q_chunk || !K_cache || !prior_len || !chunk_len || !qbar || !kbar || !scores || !mask ||
      !T || !len)
    return CA_ERR_NULL;
  if (dtype != CA_F32 && dtype != CA_BF16) return CA_ERR_DTYPE;
  if (B < 1 || B > CA_MAX_BATCH || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || C_max < 1 ||
      L < 1 || NQ_max < 1 || NKB_max < 1 || NKB_max > kMaxUnionBlocks || budget < 0 || local < 0)
    return CA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H_q * NQ_max > INT32_MAX ||
      static_cast<int64_t>(B) * H_kv > 65535)
    return CA_ERR_SHAPE;
  if (D != 64 && D != 128) return CA_ERR_UNSUPPORTED;
  if (!aligned16(Q_chunk) || !aligned16(K_cache) || !aligned16(qbar) || !aligned16(kbar))
    return CA_ERR_UNSUPPORTED;
  ca::SeqInfo seq;
  memset(&seq, 0, sizeof(seq));
  int max_pblk = 0, max_nq = 0;
  ca::SelLens dl;
  if (dev_lengths) {
    if ((reinterpret_cast<uintptr_t>(prior_len) & 3) != 0 ||
        (reinterpret_cast<uintptr_t>(chunk_len) & 3) != 0)
      return CA_ERR_UNSUPPORTED;
    dl.prior = prior_len;
    dl.chunk = chunk_len;
    dl.chunk_cap = static_cast<int>(std::min<int64_t>(C_max, static_cast<int64_t>(NQ_max) * CA_BLOCK));
    dl.total_cap = std::min<int64_t>(L, static_cast<int64_t>(NKB_max) * CA_BLOCK);
    for (int b = 0; b < B; ++b) seq.order[b] = b;
    // the largest extents the caps allow: the grids do not depend on the lengths
    max_nq = dl.chunk_cap / CA_BLOCK;
    max_pblk = static_cast<int>(dl.total_cap / CA_BLOCK);
  } else {
    for (int b = 0; b < B; ++b) {
      const int64_t P = prior_len[b], C = chunk_len[b];
      if (P < 0 || C < 0 || C > C_max || C > static_cast<int64_t>(NQ_max) * CA_BLOCK ||
          P + C > L || P + C > static_cast<int64_t>(NKB_max) * CA_BLOCK)
        return CA_ERR_SHAPE;
      if (P % CA_BLOCK != 0 || C % CA_BLOCK != 0) return CA_ERR_UNSUPPORTED;
      seq.prior[b] = static_cast<int32_t>(P);
      seq.chunk[b] = static_cast<int32_t>(C);
      seq.order[b] = b;
      max_pblk = std::max(max_pblk, static_cast<int>(P / CA_BLOCK));
      max_nq = std::max(max_nq, static_cast<int>(C / CA_BLOCK));
    }
  }
  const int64_t n_pool =
      static_cast<int64_t>(B) * (H_q + (app ? 2 : 1) * H_kv) * max_nq + B * H_kv;
  if (n_pool > INT32_MAX) return CA_ERR_SHAPE;
  return hip_status(ca::launch_select_chunk(Q_chunk, K_cache, dtype == CA_BF16 ? 2 : 4, B, H_q,
                                            H_kv, C_max, L, D, seq, max_nq, max_pblk, budget,
                                            local, qbar, NQ_max, kbar, NKB_max, scores, mask, T,
                                            len, app, dl, stream));
}

}  // namespace

extern "C" {

CA_EXPORT ca_status ca_select_chunk(const void* Q_chunk, const void* K_cache, ca_dtype dtype,
                                    int B, int H_q, int H_kv, int C_max, int64_t L, int D,
                                    const int32_t* prior_len, const int32_t* chunk_len,
                                    int budget, int local, float* qbar, int NQ_max, float* kbar,
                                    int NKB_max, float* scores, uint8_t* mask, int32_t* T,
                                    int32_t* len, hipStream_t stream) {
  return select_chunk_common(Q_chunk, K_cache, dtype, B, H_q, H_kv, C_max, L, D, prior_len,
                             chunk_len, budget, local, qbar, NQ_max, kbar, NKB_max, scores, mask,
                             T, len, nullptr, false, stream);
}

CA_EXPORT ca_status ca_select_chunk_devlen(const void* Q_chunk, const void* K_cache,
                                           ca_dtype dtype, int B, int H_q, int H_kv, int C_max,
                                           int64_t L, int D, const int32_t* prior_len,
                                           const int32_t* chunk_len, int budget, int local,
                                           float* qbar, int NQ_max, float* kbar, int NKB_max,
                                           float* scores, uint8_t* mask, int32_t* T,
                                           int32_t* len, hipStream_t stream) {
  return select_chunk_common(Q_chunk, K_cache, dtype, B, H_q, H_kv, C_max, L, D, prior_len,
                             chunk_len, budget, local, qbar, NQ_max, kbar, NKB_max, scores, mask,
                             T, len, nullptr, true, stream);
}

CA_EXPORT ca_status ca_append_select_chunk(const void* K_new, const void* V_new,
                                           const void* Q_chunk, void* K_cache, void* V_cache,
                                           ca_dtype dtype, int B, int H_q, int H_kv, int C_max,
                                           int64_t L, int D, const int32_t* prior_len,
                                           const int32_t* chunk_len, int budget, int local,
                                           float* qbar, int NQ_max, float* kbar, int NKB_max,
                                           float* scores, uint8_t* mask, int32_t* T,
                                           int32_t* len, hipStream_t stream) {
  if (!K_new || !V_new || !V_cache) return CA_ERR_NULL;
  if (!aligned16(K_new) || !aligned16(V_new) || !aligned16(V_cache)) return CA_ERR_UNSUPPORTED;
  const ca::AppendSrc app{K_new, V_new, K_cache, V_cache};
  return select_chunk_common(Q_chunk, K_cache, dtype, B, H_q, H_kv, C_max, L, D, prior_len,
                             chunk_len, budget, local, qbar, NQ_max, kbar, NKB_max, scores, mask,
                             T, len, &app, false, stream);
}

CA_EXPORT ca_status ca_append_select_chunk_devlen(
    const void* K_new, const void* V_new, const void* Q_chunk, void* K_cache, void* V_cache,
    ca_dtype dtype, int B, int H_q, int H_kv, int C_max, int64_t L, int D,
    const int32_t* prior_len, const int32_t* chunk_len, int budget, int local, float* qbar,
    int NQ_max, float* kbar, int NKB_max, float* scores, uint8_t* mask, int32_t* T, int32_t* len,
    hipStream_t stream) {
  if (!K_new || !V_new || !V_cache) return CA_ERR_NULL;
  if (!aligned16(K_new) || !aligned16(V_new) || !aligned16(V_cache)) return CA_ERR_UNSUPPORTED;
  const ca::AppendSrc app{K_new, V_new, K_cache, V_cache};
  return select_chunk_common(Q_chunk, K_cache, dtype, B, H_q, H_kv, C_max, L, D, prior_len,
                             chunk_len, budget, local, qbar, NQ_max, kbar, NKB_max, scores, mask,
                             T, len, &app, true, stream);
}

}  // extern "C"
