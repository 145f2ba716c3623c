// Explicit KV compaction: the baseline that zero-copy paged execution is
// measured against.  CompactAttention, abstract: the block tables let the
// attention read selected KV blocks in place; gathering them into a compact
// buffer first is the KV copy that this avoids.
//
// Grid (B*H_kv, kSplit): workgroup (u, s) first counts the prior blocks of
// T[u] (entries below prior/64) with a workgroup reduction, then copies blocks
// j = s, s + kSplit, ... of the table: K and V, 16-byte loads and stores over
// the whole block (HBM-bound: each selected block is read once and written
// once).

#include "kernels.hpp"

namespace ca {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kSplit = 64;  // workgroups per (b, g)

__global__ __launch_bounds__(kCopyThreads) void compact_kv_kernel(
    const uint4* __restrict__ K, const uint4* __restrict__ V, const int32_t* __restrict__ T,
    const int32_t* __restrict__ len, int NKB_max, int H_kv, int64_t slice_vec, int block_vec,
    SeqInfo seq, uint4* __restrict__ Ko, uint4* __restrict__ Vo, int32_t* __restrict__ To) {
  __shared__ int part[kCopyThreads / 64];
  const int u = blockIdx.x;
  const int s = blockIdx.y;
  const int b = u / H_kv;
  const int tid = threadIdx.x;
  const int P_blk = seq.prior[b] / 64;
  const int nkb = (seq.prior[b] + seq.chunk[b] + 63) / 64;
  int n = len[u];
  n = n < 0 ? 0 : (n > NKB_max ? NKB_max : n);
  const int32_t* trow = T + static_cast<size_t>(u) * NKB_max;
  int32_t* orow = To + static_cast<size_t>(u) * NKB_max;

  // p = number of prior blocks among the table's entries
  int cnt = 0;
  for (int j = tid; j < n; j += kCopyThreads) {
    const int kb = trow[j];
    cnt += (kb >= 0 && kb < P_blk) ? 1 : 0;
  }
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  if ((tid & 63) == 0) part[tid >> 6] = cnt;
  __syncthreads();
  int p = 0;
  for (int i = 0; i < kCopyThreads / 64; ++i) p += part[i];

  const size_t base = static_cast<size_t>(u) * slice_vec;
  for (int j = s; j < NKB_max; j += kSplit) {
    int dst = -1;
    if (j < n) {
      const int kb = trow[j];
      if (kb >= 0 && kb < nkb) {
        const int d = kb < P_blk ? P_blk - p + j : kb;
        if (d >= 0 && d < nkb) dst = d;
      }
      if (dst >= 0) {
        const uint4* ks = K + base + static_cast<size_t>(trow[j]) * block_vec;
        const uint4* vs = V + base + static_cast<size_t>(trow[j]) * block_vec;
        uint4* kd = Ko + base + static_cast<size_t>(dst) * block_vec;
        uint4* vd = Vo + base + static_cast<size_t>(dst) * block_vec;
        for (int i = tid; i < block_vec; i += kCopyThreads) {
          kd[i] = ks[i];
          vd[i] = vs[i];
        }
      }
    }
    if (tid == 0) orow[j] = dst;
  }
}

}  // namespace

hipError_t launch_compact_kv(const void* K, const void* V, const int32_t* T, const int32_t* len,
                             int NKB_max, int B, int H_kv, int64_t L, int D, int esz,
                             const SeqInfo& seq, void* Ko, void* Vo, int32_t* To,
                             hipStream_t stream) {
  const int block_vec = 64 * D * esz / 16;
  const int64_t slice_vec = L * D * esz / 16;
  hipLaunchKernelGGL(compact_kv_kernel, dim3(B * H_kv, kSplit), dim3(kCopyThreads), 0, stream,
                     static_cast<const uint4*>(K), static_cast<const uint4*>(V), T, len, NKB_max,
                     H_kv, slice_vec, block_vec, seq, static_cast<uint4*>(Ko),
                     static_cast<uint4*>(Vo), To);
  return hipGetLastError();
}

}  // namespace ca
