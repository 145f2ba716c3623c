// Block-Union KV selection on gfx950.
//
// CompactAttention, selection stage ("Methodology" of the technical summaries;
// abstract): the per-head 2D block mask is reduced over the chunk's Q-blocks
// (Q-block union) and over the query heads that share a KV head (intra-group
// union).  The result T[b,g] is the minimal table that keeps every selected KV
// block: exactly the set union, written strictly ascending and padded with -1.
//
// One workgroup (1024 threads, 16 waves) per pseudo-request (b, g):
//   1. OR-reduce: each thread ORs 16-byte slices of the G * n_q_blocks mask rows
//      of its column range in registers (threads split the rows when the
//      columns alone cannot occupy the workgroup), turns nonzero bytes into
//      bits and ORs them into an LDS bitmap of NKB_max bits.
//   2. Compaction: each thread owns a contiguous run of bitmap words; a
//      workgroup prefix sum of their popcounts (per wave from ballots of the
//      count's bit planes, then across the 16 waves) gives each thread its
//      output offset, so block ids come out in ascending order.
// The mask is read once (HBM-bound, one pass); everything else stays on chip.

#include "kernels.hpp"

namespace ca {
namespace {

constexpr int kUnionThreads = 1024;
constexpr int kUnionWaves = kUnionThreads / 64;

// Exclusive prefix sum of v over the 64 lanes of a wave, from one ballot per
// bit plane of v (v >= 0).  All lanes must call it.
__device__ inline int wave_exclusive_prefix(int v) {
  int r = 0;
  for (int k = 0; k < 31; ++k) {
    if (__ballot((v >> k) != 0) == 0) break;  // no lane has bits >= k left
    const uint64_t bal = __ballot((v >> k) & 1);
    const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
    r += below << k;
  }
  return r;
}

// Nonzero bytes of x -> low 4 bits (bit j set iff byte j != 0).
__device__ inline uint32_t nonzero_bytes4(uint32_t x) {
  const uint32_t hi = ((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x;  // bit 7 of each byte = byte != 0
  return ((hi >> 7) & 1u) | ((hi >> 14) & 2u) | ((hi >> 21) & 4u) | ((hi >> 28) & 8u);
}

template <int VW>  // bytes per load: 16 (rows 16-byte aligned) or 1
__global__ __launch_bounds__(kUnionThreads) void union_tables_kernel(
    const uint8_t* __restrict__ mask, int H_q, int H_kv, int NQ_max, int NKB_max,
    UnionExtents ext, const int32_t* __restrict__ dev_nq, const int32_t* __restrict__ dev_nkb,
    int32_t* __restrict__ T, int32_t* __restrict__ len) {
  extern __shared__ uint32_t bitmap[];  // ceil(NKB_max / 32) words
  __shared__ int wave_total[kUnionWaves];

  const int bg = blockIdx.x;
  const int b = bg / H_kv;
  const int g = bg - b * H_kv;
  const int G = H_q / H_kv;
  int nq = ext.nq[b];
  int nkb = ext.nkb[b];
  if (dev_nq != nullptr) {  // device extents: out of range -> an empty table
    nq = dev_nq[b];
    nkb = dev_nkb[b];
    if (nq < 0 || nq > NQ_max || nkb < 0 || nkb > NKB_max) nq = nkb = 0;
  }
  const int tid = threadIdx.x;
  const int nwords = (NKB_max + 31) >> 5;

  for (int w = tid; w < nwords; w += kUnionThreads) bitmap[w] = 0u;
  __syncthreads();

  // ---- 1. OR over the group's heads and the chunk's Q-blocks
  const int rows = G * nq;
  const int nchunks = (nkb + VW - 1) / VW;
  if (rows > 0 && nchunks > 0) {
    int rgroups = kUnionThreads / nchunks;
    rgroups = rgroups < 1 ? 1 : (rgroups > rows ? rows : rgroups);
    const size_t head0 = static_cast<size_t>(b) * H_q + static_cast<size_t>(g) * G;
    for (int item = tid; item < nchunks * rgroups; item += kUnionThreads) {
      const int ch = item % nchunks;
      const int rg = item / nchunks;
      uint32_t bits = 0;
      if constexpr (VW == 16) {
        auto slice = [&](int r) {  // 16 bytes of mask row r (head hg of the group, Q-block qb)
          const int hg = r / nq;
          const int qb = r - hg * nq;
          const uint8_t* row = mask + ((head0 + hg) * NQ_max + qb) * static_cast<size_t>(NKB_max);
          return *reinterpret_cast<const uint4*>(row + static_cast<size_t>(ch) * 16);
        };
        uint4 acc = make_uint4(0u, 0u, 0u, 0u);
        // eight rows' loads in flight before any is combined: the reduction is
        // bound by memory latency, not bandwidth, at these sizes
        constexpr int kBatch = 8;
        int r = rg;
        for (; r + (kBatch - 1) * rgroups < rows; r += kBatch * rgroups) {
          uint4 x[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) x[u] = slice(r + u * rgroups);
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            acc.x |= x[u].x; acc.y |= x[u].y; acc.z |= x[u].z; acc.w |= x[u].w;
          }
        }
        for (; r < rows; r += rgroups) {
          const uint4 x = slice(r);
          acc.x |= x.x; acc.y |= x.y; acc.z |= x.z; acc.w |= x.w;
        }
        bits = nonzero_bytes4(acc.x) | (nonzero_bytes4(acc.y) << 4) |
               (nonzero_bytes4(acc.z) << 8) | (nonzero_bytes4(acc.w) << 12);
        const int valid = nkb - ch * 16;  // columns >= nkb are outside the sequence
        if (valid < 16) bits &= (1u << valid) - 1u;
      } else {
        uint32_t acc = 0;
        for (int r = rg; r < rows; r += rgroups) {
          const int hg = r / nq;
          const int qb = r - hg * nq;
          acc |= mask[((head0 + hg) * NQ_max + qb) * static_cast<size_t>(NKB_max) + ch];
        }
        bits = acc != 0u ? 1u : 0u;
      }
      if (bits) atomicOr(&bitmap[(ch * VW) >> 5], bits << ((ch * VW) & 31));
    }
  }
  __syncthreads();

  // ---- 2. ascending compaction by a workgroup prefix sum of popcounts
  const int wpt = (nwords + kUnionThreads - 1) / kUnionThreads;
  const int w0 = min(tid * wpt, nwords);
  const int w1 = min(w0 + wpt, nwords);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bitmap[w]);
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int excl = wave_exclusive_prefix(cnt);
  if (lane == 63) wave_total[wave] = excl + cnt;
  __syncthreads();
  int base = 0, total = 0;
  for (int i = 0; i < kUnionWaves; ++i) {
    const int t = wave_total[i];
    base += (i < wave) ? t : 0;
    total += t;
  }
  int32_t* trow = T + static_cast<size_t>(bg) * NKB_max;
  int off = base + excl;
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bitmap[w];
    while (m) {
      const int j = __ffs(m) - 1;
      trow[off++] = (w << 5) + j;
      m &= m - 1u;
    }
  }
  for (int j = total + tid; j < NKB_max; j += kUnionThreads) trow[j] = -1;
  if (tid == 0) len[bg] = total;
}

// One workgroup per pseudo-request u: its offset is the sum of the earlier
// lengths (reduced in the workgroup), then its block ids become page ids.
constexpr int kCsrThreads = 256;

__global__ __launch_bounds__(kCsrThreads) void tables_to_csr_kernel(
    const int32_t* __restrict__ T, const int32_t* __restrict__ len, int n_bg, int NKB_max,
    int64_t pages, int32_t* __restrict__ kv_indptr, int32_t* __restrict__ kv_indices) {
  __shared__ int partial[kCsrThreads / 64];
  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  auto clamp_len = [&](int x) { return x < 0 ? 0 : (x > NKB_max ? NKB_max : x); };
  int s = 0;
  for (int i = tid; i < u; i += kCsrThreads) s += clamp_len(len[i]);
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((tid & 63) == 0) partial[tid >> 6] = s;
  __syncthreads();
  int off = 0;
  for (int i = 0; i < kCsrThreads / 64; ++i) off += partial[i];
  const int n = clamp_len(len[u]);
  if (tid == 0) {
    kv_indptr[u] = off;
    if (u == n_bg - 1) kv_indptr[n_bg] = off + n;
  }
  const int32_t* trow = T + static_cast<size_t>(u) * NKB_max;
  const int64_t page0 = static_cast<int64_t>(u) * pages;
  for (int j = tid; j < n; j += kCsrThreads)
    kv_indices[off + j] = static_cast<int32_t>(page0 + trow[j]);
}

// Contract check of one table row (the properties chunk attention relies on
// without checking them on the device): one workgroup per pseudo-request, a
// bitmask of the violations found (see ca_check_tables).
constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void check_tables_kernel(
    const int32_t* __restrict__ T, const int32_t* __restrict__ len, int H_kv, int NKB_max,
    UnionExtents ext, int32_t* __restrict__ row_bad) {
  __shared__ int flags[kCheckThreads / 64];
  const int bg = blockIdx.x;
  const int b = bg / H_kv;
  const int tid = threadIdx.x;
  const int nkb = ext.nkb[b];
  const int n = len[bg];
  int f = (n < 0 || n > NKB_max) ? 1 : 0;
  const int nc = n < 0 ? 0 : (n > NKB_max ? NKB_max : n);
  const int32_t* trow = T + static_cast<size_t>(bg) * NKB_max;
  for (int j = tid; j < NKB_max; j += kCheckThreads) {
    const int v = trow[j];
    if (j < nc) {
      if (v < 0 || v >= nkb) f |= 2;
      if (j > 0 && v <= trow[j - 1]) f |= 4;
    } else if (v != -1) {
      f |= 8;
    }
  }
  // OR over the workgroup: per wave through its lanes, then across waves
  for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o);
  if ((tid & 63) == 0) flags[tid >> 6] = f;
  __syncthreads();
  if (tid == 0) {
    int all = 0;
    for (int w = 0; w < kCheckThreads / 64; ++w) all |= flags[w];
    row_bad[bg] = all;
  }
}

}  // namespace

hipError_t launch_union_tables(const uint8_t* mask, int B, int H_q, int H_kv, int NQ_max,
                               int NKB_max, const UnionExtents& ext, const int32_t* dev_nq,
                               const int32_t* dev_nkb, int32_t* T, int32_t* len,
                               hipStream_t stream) {
  const size_t lds = static_cast<size_t>((NKB_max + 31) / 32) * sizeof(uint32_t);
  const bool vec = (NKB_max % 16 == 0) && (reinterpret_cast<uintptr_t>(mask) % 16 == 0);
  dim3 grid(B * H_kv), block(kUnionThreads);
  if (vec)
    hipLaunchKernelGGL(union_tables_kernel<16>, grid, block, lds, stream, mask, H_q, H_kv,
                       NQ_max, NKB_max, ext, dev_nq, dev_nkb, T, len);
  else
    hipLaunchKernelGGL(union_tables_kernel<1>, grid, block, lds, stream, mask, H_q, H_kv,
                       NQ_max, NKB_max, ext, dev_nq, dev_nkb, T, len);
  return hipGetLastError();
}

hipError_t launch_check_tables(const int32_t* T, const int32_t* len, int n_bg, int H_kv,
                               int NKB_max, const UnionExtents& ext, int32_t* row_bad,
                               hipStream_t stream) {
  hipLaunchKernelGGL(check_tables_kernel, dim3(n_bg), dim3(kCheckThreads), 0, stream, T, len,
                     H_kv, NKB_max, ext, row_bad);
  return hipGetLastError();
}

hipError_t launch_tables_to_csr(const int32_t* T, const int32_t* len, int n_bg, int NKB_max,
                                int64_t pages, int32_t* kv_indptr, int32_t* kv_indices,
                                hipStream_t stream) {
  hipLaunchKernelGGL(tables_to_csr_kernel, dim3(n_bg), dim3(kCsrThreads), 0, stream, T, len,
                     n_bg, NKB_max, pages, kv_indptr, kv_indices);
  return hipGetLastError();
}

}  // namespace ca
