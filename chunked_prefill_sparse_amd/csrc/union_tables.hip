// Block-Union KV selection on gfx950.
//
// CompactAttention, selection stage ("Methodology" of the technical summaries;
// abstract): the per-head 2D block mask is reduced over the chunk's Q-blocks
// (Q-block union) and over the query heads that share a KV head (intra-group
// union).  The result T[b,g] is the minimal table that keeps every selected KV
// block: exactly the set union, written strictly ascending and padded with -1.
//
// Two steps per pseudo-request (b, g):
//   1. OR-reduce: 16-byte slices of the G * n_q_blocks mask rows are ORed in
//      registers (threads split the rows when the columns alone cannot occupy
//      the workgroup), nonzero bytes become bits, and the bits are ORed into an
//      LDS bitmap with atomicOr.
//   2. Compaction: each thread owns a contiguous run of bitmap words; a
//      workgroup prefix sum of their popcounts (per wave from ballots of the
//      count's bit planes, then across the waves) gives each thread its output
//      offset, so block ids come out in ascending order.
// When there are many pseudo-requests (or rows are not 16-byte aligned), one
// workgroup does both for one (b, g).  When there are few (a single 128K
// sequence has 8), one workgroup per (b, g) would leave most of the chip idle
// while it streams 256 KiB of mask, so step 1 is spread over column slices,
// one workgroup each: a slice's bitmap words are parked in the tail of the
// T[b,g] row (ceil(NKB_max / 32) of its NKB_max entries), and a second kernel
// compacts them, one workgroup per (b, g), after loading the words into LDS.
// The mask is read once (HBM-bound, one pass); everything else stays on chip.

#include "kernels.hpp"

namespace ca {
namespace {

constexpr int kUnionThreads = 1024;
constexpr int kUnionWaves = kUnionThreads / 64;
constexpr int kMaxSliceCols = 8192;  // columns per slice of the sliced OR step

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

// Extents of sequence b: the host values, or (device-length calls) the device
// values, checked here (out of range -> an empty table).
__device__ inline void union_extents(const UnionExtents& ext, const int32_t* dev_nq,
                                     const int32_t* dev_nkb, int b, int NQ_max, int NKB_max,
                                     int& nq, int& nkb) {
  nq = ext.nq[b];
  nkb = ext.nkb[b];
  if (dev_nq != nullptr) {
    nq = dev_nq[b];
    nkb = dev_nkb[b];
    if (nq < 0 || nq > NQ_max || nkb < 0 || nkb > NKB_max) nq = nkb = 0;
  }
}

// 16 bits of 16 mask columns: bit j set iff byte j of the ORed slice is nonzero.
__device__ inline uint32_t nonzero_bytes16(const uint4& a) {
  return nonzero_bytes4(a.x) | (nonzero_bytes4(a.y) << 4) | (nonzero_bytes4(a.z) << 8) |
         (nonzero_bytes4(a.w) << 12);
}

// OR of 16-byte column chunk `ch` over the rows r = r0, r0 + rstep, ... < rows
// of a group (row r = head r / nq of the group, Q-block r % nq), with eight
// rows' loads in flight before any is combined: the reduction is bound by
// memory latency, not bandwidth, at these sizes.
__device__ inline uint4 or_rows16(const uint8_t* __restrict__ mask, size_t head0, int nq,
                                  int NQ_max, int NKB_max, int ch, int r0, int rstep, int rows) {
  auto slice = [&](int r) {
    const int hg = r / nq;
    const int qb = r - hg * nq;
    const uint8_t* row = mask + ((head0 + hg) * NQ_max + qb) * static_cast<size_t>(NKB_max);
    return *reinterpret_cast<const uint4*>(row + static_cast<size_t>(ch) * 16);
  };
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  constexpr int kBatch = 8;
  int r = r0;
  for (; r + (kBatch - 1) * rstep < rows; r += kBatch * rstep) {
    uint4 x[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) x[u] = slice(r + u * rstep);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      acc.x |= x[u].x; acc.y |= x[u].y; acc.z |= x[u].z; acc.w |= x[u].w;
    }
  }
  for (; r < rows; r += rstep) {
    const uint4 x = slice(r);
    acc.x |= x.x; acc.y |= x.y; acc.z |= x.z; acc.w |= x.w;
  }
  return acc;
}

// Ascending compaction of an LDS bitmap of nwords words into the T row (then
// -1 up to NKB_max) and its length, by a workgroup prefix sum of popcounts.
// The bitmap must be complete (barrier) before the call.
template <int kThreads>
__device__ inline void compact_bitmap(const uint32_t* bitmap, int nwords, int NKB_max,
                                      int32_t* __restrict__ trow, int32_t* __restrict__ len_out,
                                      int* wave_total) {
  constexpr int kWaves = kThreads / 64;
  const int tid = threadIdx.x;
  const int wpt = (nwords + kThreads - 1) / kThreads;
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
  for (int i = 0; i < kWaves; ++i) {
    const int t = wave_total[i];
    base += (i < wave) ? t : 0;
    total += t;
  }
  int off = base + excl;
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bitmap[w];
    while (m) {
      const int j = __ffs(m) - 1;
      trow[off++] = (w << 5) + j;
      m &= m - 1u;
    }
  }
  for (int j = total + tid; j < NKB_max; j += kThreads) trow[j] = -1;
  if (tid == 0) *len_out = total;
}

// Both steps for one pseudo-request per workgroup.
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
  int nq, nkb;
  union_extents(ext, dev_nq, dev_nkb, b, NQ_max, NKB_max, nq, nkb);
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
        bits = nonzero_bytes16(or_rows16(mask, head0, nq, NQ_max, NKB_max, ch, rg, rgroups,
                                         rows));
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
  compact_bitmap<kUnionThreads>(bitmap, nwords, NKB_max, T + static_cast<size_t>(bg) * NKB_max,
                                len + bg, wave_total);
}

// Step 1 over column slices (rows 16-byte aligned): workgroup (u, s) ORs
// columns [s * slice, (s + 1) * slice) of pseudo-request u's rows and parks its
// bitmap words w (global word index) at T[u, NKB_max - nwords + w].
constexpr int kSliceThreads = 256;

__global__ __launch_bounds__(kSliceThreads) void union_slice_kernel(
    const uint8_t* __restrict__ mask, int H_q, int H_kv, int NQ_max, int NKB_max, int slice,
    int n_slices, UnionExtents ext, const int32_t* __restrict__ dev_nq,
    const int32_t* __restrict__ dev_nkb, int32_t* __restrict__ T) {
  __shared__ uint32_t words[kMaxSliceCols / 32];
  const int u = blockIdx.x / n_slices;
  const int sl = blockIdx.x - u * n_slices;
  const int b = u / H_kv;
  const int g = u - b * H_kv;
  const int G = H_q / H_kv;
  int nq, nkb;
  union_extents(ext, dev_nq, dev_nkb, b, NQ_max, NKB_max, nq, nkb);
  const int tid = threadIdx.x;
  const int c0 = sl * slice;
  const int c1 = min(c0 + slice, NKB_max);
  const int nw = (c1 - c0 + 31) >> 5;
  for (int w = tid; w < nw; w += kSliceThreads) words[w] = 0u;
  __syncthreads();
  const int rows = G * nq;
  const int ce = min(c1, nkb);  // columns >= nkb are outside the sequence
  const int nch = ce > c0 ? (ce - c0 + 15) / 16 : 0;
  if (rows > 0 && nch > 0) {
    int rgroups = kSliceThreads / nch;
    rgroups = rgroups < 1 ? 1 : (rgroups > rows ? rows : rgroups);
    const size_t head0 = static_cast<size_t>(b) * H_q + static_cast<size_t>(g) * G;
    for (int item = tid; item < nch * rgroups; item += kSliceThreads) {
      const int k = item % nch;
      const int rg = item / nch;
      const int ch = c0 / 16 + k;
      uint32_t bits = nonzero_bytes16(or_rows16(mask, head0, nq, NQ_max, NKB_max, ch, rg,
                                                rgroups, rows));
      const int valid = nkb - ch * 16;
      if (valid < 16) bits &= (1u << valid) - 1u;
      if (bits) atomicOr(&words[(k * 16) >> 5], bits << ((k * 16) & 31));
    }
  }
  __syncthreads();
  const int nwords = (NKB_max + 31) >> 5;
  int32_t* tail = T + static_cast<size_t>(u) * NKB_max + (NKB_max - nwords) + (c0 >> 5);
  for (int w = tid; w < nw; w += kSliceThreads) tail[w] = static_cast<int32_t>(words[w]);
}

// Step 2 after union_slice_kernel: load the parked words of row u into LDS,
// then compact them over the whole row.
// n_rep copies of the bitmap lie side by side at the tail (the fused selection
// spreads its atomics over them); they are ORed together.
template <int kThreads>  // 256 for bitmaps of up to 256 words (8192 blocks), else 1024
__global__ __launch_bounds__(kThreads) void union_compact_kernel(
    int NKB_max, int n_rep, int32_t* __restrict__ T, int32_t* __restrict__ len) {
  extern __shared__ uint32_t bitmap[];  // ceil(NKB_max / 32) words
  __shared__ int wave_total[kThreads / 64];
  const int u = blockIdx.x;
  const int nwords = (NKB_max + 31) >> 5;
  int32_t* trow = T + static_cast<size_t>(u) * NKB_max;
  const int32_t* tail = trow + NKB_max - n_rep * nwords;
  if (n_rep == 1) {
    for (int w = threadIdx.x; w < nwords; w += kThreads) bitmap[w] = static_cast<uint32_t>(tail[w]);
  } else {
    const int total = n_rep * nwords;
    for (int w = threadIdx.x; w < nwords; w += kThreads) bitmap[w] = 0u;
    __syncthreads();
    for (int base = 0; base < total; base += 4 * kThreads) {
      uint32_t x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // clamped index: the four loads go out together
        const int i = base + j * kThreads + static_cast<int>(threadIdx.x);
        x[j] = static_cast<uint32_t>(tail[i < total ? i : total - 1]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = base + j * kThreads + static_cast<int>(threadIdx.x);
        if (i < total && x[j] != 0u) atomicOr(&bitmap[i % nwords], x[j]);
      }
    }
  }
  __syncthreads();  // every parked word is in LDS before the row is overwritten
  compact_bitmap<kThreads>(bitmap, nwords, NKB_max, trow, len + u, wave_total);
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
                               const int32_t* dev_nkb, int32_t* T, int32_t* len, int cus,
                               hipStream_t stream) {
  const size_t lds = static_cast<size_t>((NKB_max + 31) / 32) * sizeof(uint32_t);
  const bool vec = (NKB_max % 16 == 0) && (reinterpret_cast<uintptr_t>(mask) % 16 == 0);
  const int n_bg = B * H_kv;
  // column slices of 256 (whole words) up to kMaxSliceCols, about one
  // workgroup per compute unit over all pseudo-requests (measured at 128K, in
  // graph replay: 6.3 us per call with 256-column slices, 6.6 with 128, 8.5
  // with one workgroup per (b, g))
  int n_slices = 1;
  if (vec && n_bg < cus) {
    const int want = (cus + n_bg - 1) / n_bg;
    int slice = (NKB_max + want - 1) / want;
    slice = (slice + 255) / 256 * 256;
    slice = slice < kMaxSliceCols ? slice : kMaxSliceCols;
    n_slices = (NKB_max + slice - 1) / slice;
    if (n_slices > 1) {
      hipLaunchKernelGGL(union_slice_kernel, dim3(n_bg * n_slices), dim3(kSliceThreads), 0,
                         stream, mask, H_q, H_kv, NQ_max, NKB_max, slice, n_slices, ext, dev_nq,
                         dev_nkb, T);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_union_compact(n_bg, NKB_max, 1, T, len, stream);
    }
  }
  dim3 grid(n_bg), block(kUnionThreads);
  if (vec)
    hipLaunchKernelGGL(union_tables_kernel<16>, grid, block, lds, stream, mask, H_q, H_kv,
                       NQ_max, NKB_max, ext, dev_nq, dev_nkb, T, len);
  else
    hipLaunchKernelGGL(union_tables_kernel<1>, grid, block, lds, stream, mask, H_q, H_kv,
                       NQ_max, NKB_max, ext, dev_nq, dev_nkb, T, len);
  return hipGetLastError();
}

hipError_t launch_union_compact(int n_bg, int NKB_max, int n_rep, int32_t* T, int32_t* len,
                                hipStream_t stream) {
  const size_t lds = static_cast<size_t>((NKB_max + 31) / 32) * sizeof(uint32_t);
  if ((NKB_max + 31) / 32 <= 256)
    hipLaunchKernelGGL(union_compact_kernel<256>, dim3(n_bg), dim3(256), lds, stream, NKB_max,
                       n_rep, T, len);
  else
    hipLaunchKernelGGL(union_compact_kernel<kUnionThreads>, dim3(n_bg), dim3(kUnionThreads), lds,
                       stream, NKB_max, n_rep, T, len);
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
