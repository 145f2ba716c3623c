// Append of one chunk's keys and values to the KV-head-major cache.
//
// Chunked prefill (CompactAttention, problem statement of the technical
// summaries): a long prompt is processed chunk by chunk, and each chunk
// attends to the cache accumulated so far plus itself, so its own keys and
// values are written into the cache first, at rows [prior, prior + chunk) of
// every (sequence, KV head) slice.  A plain HBM-bound copy: 16-byte loads,
// all of a thread's loads in flight before its stores.

#include "kernels.hpp"

namespace ca {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kAppendVec = 4;  // 16-byte vectors per thread

// Workgroup (u = b * H_kv + g, y, z): vectors [y * 1024, (y + 1) * 1024) of
// the chunk rows of slice u, of K (z = 0) or V (z = 1).
__global__ __launch_bounds__(kAppendThreads) void append_kv_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new, int H_kv,
    int64_t new_slice_vec, int64_t cache_slice_vec, int row_vec, SeqInfo seq,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache) {
  const int u = blockIdx.x;
  const int b = u / H_kv;
  const int64_t n = static_cast<int64_t>(seq.chunk[b]) * row_vec;  // vectors to copy
  const int64_t i0 = static_cast<int64_t>(blockIdx.y) * kAppendThreads * kAppendVec + threadIdx.x;
  const uint4* src = (blockIdx.z == 0 ? k_new : v_new) + static_cast<int64_t>(u) * new_slice_vec;
  uint4* dst = (blockIdx.z == 0 ? k_cache : v_cache) + static_cast<int64_t>(u) * cache_slice_vec +
               static_cast<int64_t>(seq.prior[b]) * row_vec;
  uint4 x[kAppendVec];
  const int64_t wg_end = (static_cast<int64_t>(blockIdx.y) + 1) * kAppendThreads * kAppendVec;
  if (wg_end <= n) {
    // whole workgroup in range (uniform): unguarded loads, so all four are in
    // flight before the first wait (guarded ones each wait on their own)
#pragma unroll
    for (int k = 0; k < kAppendVec; ++k) x[k] = src[i0 + static_cast<int64_t>(k) * kAppendThreads];
#pragma unroll
    for (int k = 0; k < kAppendVec; ++k) dst[i0 + static_cast<int64_t>(k) * kAppendThreads] = x[k];
    return;
  }
#pragma unroll
  for (int k = 0; k < kAppendVec; ++k) {
    const int64_t i = i0 + static_cast<int64_t>(k) * kAppendThreads;
    if (i < n) x[k] = src[i];
  }
#pragma unroll
  for (int k = 0; k < kAppendVec; ++k) {
    const int64_t i = i0 + static_cast<int64_t>(k) * kAppendThreads;
    if (i < n) dst[i] = x[k];
  }
}

}  // namespace

hipError_t launch_append_kv(const void* k_new, const void* v_new, int B, int H_kv, int C_max,
                            int64_t L, int D, int esz, const SeqInfo& seq, void* k_cache,
                            void* v_cache, hipStream_t stream) {
  const int row_vec = D * esz / 16;
  const int64_t per_slice = static_cast<int64_t>(C_max) * row_vec;
  const int64_t per_wg = kAppendThreads * kAppendVec;
  const dim3 grid(B * H_kv, static_cast<unsigned>((per_slice + per_wg - 1) / per_wg), 2);
  hipLaunchKernelGGL(append_kv_kernel, grid, dim3(kAppendThreads), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), H_kv,
                     per_slice, L * row_vec, row_vec, seq, static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache));
  return hipGetLastError();
}

}  // namespace ca
