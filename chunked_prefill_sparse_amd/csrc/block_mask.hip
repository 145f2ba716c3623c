// A lightweight block-mask producer on gfx950 (the step upstream of the
// union).  CompactAttention, "Methodology" (selection stage) and the problem
// statement of the technical summaries: the union takes a per-head 2D block
// mask from whatever cheap searcher the caller uses, and that search runs again over
// the growing KV cache at every chunk, so its cost matters.  The pages leave
// the searcher open; this one is training-free:
//
//   qbar[b,h,qb]  = mean of the 64 rows of Q-block qb          (pool_blocks)
//   kbar[b,g,kb]  = mean of the 64 rows of KV block kb         (pool_blocks,
//                   kept across chunks: only the new blocks are pooled)
//   s[b,h,qb,kb]  = qbar . kbar                                (block_scores,
//                   bf16 hi/lo parts of the fp32 values on the
//                   matrix cores, within 2^-14 of sum_d |q_d k_d|)
//   mask row      = sink + last `local` prior blocks + causal block triangle
//                   + the `budget` best remaining prior blocks  (topk_mask)
//
// All three are HBM/L2-bound and tiny next to the attention: pooling reads
// each new block once; the scores read kbar once per KV group; the selection
// reads each score row a few times from L2 and writes one mask byte per cell.

#include <algorithm>

#include "kernels.hpp"

namespace ca {
namespace {

constexpr int kMaskThreads = 256;
constexpr int kSelectReplicas = 16;  // union bitmap copies of the fused selection
constexpr int kTopkStage = 8;        // score loads in flight per thread when staging keys
constexpr int kTopkLdsMax = 15360;   // rows up to this many blocks stage keys in LDS (60 KiB)

// Prior and chunk length of sequence b for the selection kernels: the host
// values in SeqInfo, or (device-length calls, dl.prior != nullptr) the values
// in device memory, checked here: lengths that are negative, not multiples of
// 64, a chunk past dl.chunk_cap, or a total past dl.total_cap make an empty
// chunk (no block pooled, no row selected, an empty table).
__device__ __forceinline__ void sel_lengths(const SelLens& dl, const SeqInfo& seq, int b,
                                            int& P, int& C) {
  if (dl.prior == nullptr) {
    P = seq.prior[b];
    C = seq.chunk[b];
    return;
  }
  const int P_ = dl.prior[b];
  const int C_ = dl.chunk[b];
  const bool ok = P_ >= 0 && C_ >= 0 && ((P_ | C_) & 63) == 0 && C_ <= dl.chunk_cap &&
                  static_cast<int64_t>(P_) + C_ <= dl.total_cap;
  P = ok ? P_ : 0;
  C = ok ? C_ : 0;
}

// ---------------------------------------------------------------- pooling

// How the pooling's threads hold one 64-row block (row stride D): thread tid
// owns the 16-byte column slice (tid % TPR) * V of rows tid / TPR + k * RPI,
// k < NR, which covers the block once.
template <typename TIn, int D>
struct PoolShape {
  static constexpr int V = 16 / static_cast<int>(sizeof(TIn));  // elements per 16-byte load
  static constexpr int TPR = D / V;                              // threads per row
  static constexpr int RPI = kMaskThreads / TPR;                 // rows per iteration
  static constexpr int NR = 64 / RPI;                            // vectors per thread
  static_assert(64 % RPI == 0, "rows of a block split evenly over the row groups");
};

// This thread's NR vectors of the block at src, all loads in flight together.
template <typename TIn, int D>
__device__ __forceinline__ void load_block_vecs(const TIn* __restrict__ src, uint4* raw) {
  using S = PoolShape<TIn, D>;
  const int tid = threadIdx.x;
  const int col = (tid % S::TPR) * S::V;
  const int rsub = tid / S::TPR;
#pragma unroll
  for (int k = 0; k < S::NR; ++k)
    raw[k] = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(rsub + k * S::RPI) * D + col);
}

// The same vectors written to the block at dst (the append's copy).
template <typename TIn, int D>
__device__ __forceinline__ void store_block_vecs(TIn* __restrict__ dst, const uint4* raw) {
  using S = PoolShape<TIn, D>;
  const int tid = threadIdx.x;
  const int col = (tid % S::TPR) * S::V;
  const int rsub = tid / S::TPR;
#pragma unroll
  for (int k = 0; k < S::NR; ++k)
    *reinterpret_cast<uint4*>(dst + static_cast<size_t>(rsub + k * S::RPI) * D + col) = raw[k];
}

// Mean of the 64 rows of one block into out[0 .. D), from the vectors the
// threads hold: each thread sums its column slice over its rows, then the RPI
// partial sums of a column are added in row-group order.
template <typename TIn, int D>
__device__ __forceinline__ void pool_block_vecs(const uint4* raw, float* __restrict__ out,
                                                float* part) {
  using S = PoolShape<TIn, D>;
  const int tid = threadIdx.x;
  const int col = (tid % S::TPR) * S::V;
  const int rsub = tid / S::TPR;
  float acc[S::V];
#pragma unroll
  for (int i = 0; i < S::V; ++i) acc[i] = 0.f;
#pragma unroll
  for (int k = 0; k < S::NR; ++k) {
    const TIn* e = reinterpret_cast<const TIn*>(&raw[k]);
#pragma unroll
    for (int i = 0; i < S::V; ++i) acc[i] += static_cast<float>(e[i]);
  }
#pragma unroll
  for (int i = 0; i < S::V; ++i) part[rsub * D + col + i] = acc[i];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int k = 0; k < S::RPI; ++k) s += part[k * D + tid];
    out[tid] = s * (1.f / 64.f);
  }
}

// Mean of the 64 rows of one block (src points at its first row, row stride D).
template <typename TIn, int D>
__device__ __forceinline__ void pool_one_block(const TIn* __restrict__ src,
                                               float* __restrict__ out, float* part) {
  uint4 raw[PoolShape<TIn, D>::NR];
  load_block_vecs<TIn, D>(src, raw);
  pool_block_vecs<TIn, D>(raw, out, part);
}

template <typename TIn, int D>
constexpr int kPoolPart = (kMaskThreads / (D / (16 / static_cast<int>(sizeof(TIn))))) * D;

// Workgroup (b*H + h, y) pools block kb = begin[b] + y.
template <typename TIn, int D>
__global__ __launch_bounds__(kMaskThreads) void pool_blocks_kernel(const TIn* __restrict__ X,
                                                                   int H, int64_t R,
                                                                   BlockRange rng,
                                                                   float* __restrict__ out,
                                                                   int NB_out) {
  __shared__ float part[kPoolPart<TIn, D>];
  const int bh = blockIdx.x;
  const int b = bh / H;
  const int kb = rng.begin[b] + static_cast<int>(blockIdx.y);
  if (kb >= rng.end[b]) return;
  pool_one_block<TIn, D>(X + (static_cast<size_t>(bh) * R + static_cast<size_t>(kb) * 64) * D,
                         out + (static_cast<size_t>(bh) * NB_out + kb) * D, part);
}

// First launch of a chunk's selection: workgroup w < nK pools the chunk's new
// key block (b, g, P/64 + y) into kbar; the next nQ workgroups pool its
// Q-block (b, h, y) into qbar; the last B * H_kv workgroups clear the union
// bitmaps at the tail of each T[b,g] row (n_rep copies of ceil(NKB_max / 32)
// words), which the selection then ORs into.
// kAppend (the chunk's append fused in): the key blocks come from k_new (the
// chunk's rows, [B, H_kv, C_max, D]) and are also written to the cache at rows
// P + 64y, and nK more workgroups (after the key blocks) copy the value
// blocks of v_new the same way.  The pooled values are the same as pooling
// the cache after the append, bit for bit: the same rows, summed in the same
// order.
template <typename TIn, int D, bool kAppend>
__global__ __launch_bounds__(kMaskThreads) void select_pool_kernel(
    const TIn* __restrict__ K, const TIn* __restrict__ Q, int H_q, int H_kv, int64_t L,
    int C_max, int NQ_max, int NKB_max, int span, int n_k, int n_q, int n_rep, SeqInfo seq,
    float* __restrict__ kbar, float* __restrict__ qbar, int32_t* __restrict__ T,
    const TIn* __restrict__ k_new, const TIn* __restrict__ v_new, TIn* __restrict__ k_cache,
    TIn* __restrict__ v_cache, SelLens dl) {
  __shared__ float part[kPoolPart<TIn, D>];
  int w = blockIdx.x;  // n_k = B * H_kv * span key blocks, n_q = B * H_q * span Q-blocks
  if (w < (kAppend ? 2 * n_k : n_k)) {
    const bool is_v = w >= n_k;
    if (is_v) w -= n_k;
    const int bg = w / span, y = w - bg * span;
    const int b = bg / H_kv;
    int P, C;
    sel_lengths(dl, seq, b, P, C);
    const int kb = P / 64 + y;
    if (y >= C / 64) return;
    const size_t cache_off = (static_cast<size_t>(bg) * L + static_cast<size_t>(kb) * 64) * D;
    if constexpr (kAppend) {
      const size_t new_off = (static_cast<size_t>(bg) * C_max + static_cast<size_t>(y) * 64) * D;
      uint4 raw[PoolShape<TIn, D>::NR];
      load_block_vecs<TIn, D>((is_v ? v_new : k_new) + new_off, raw);
      store_block_vecs<TIn, D>((is_v ? v_cache : k_cache) + cache_off, raw);
      if (!is_v)
        pool_block_vecs<TIn, D>(raw, kbar + (static_cast<size_t>(bg) * NKB_max + kb) * D, part);
    } else {
      pool_one_block<TIn, D>(K + cache_off, kbar + (static_cast<size_t>(bg) * NKB_max + kb) * D,
                             part);
    }
    return;
  }
  w -= kAppend ? 2 * n_k : n_k;
  if (w < n_q) {
    const int bh = w / span, y = w - bh * span;
    const int b = bh / H_q;
    int P, C;
    sel_lengths(dl, seq, b, P, C);
    if (y >= C / 64) return;
    pool_one_block<TIn, D>(Q + (static_cast<size_t>(bh) * C_max + static_cast<size_t>(y) * 64) * D,
                           qbar + (static_cast<size_t>(bh) * NQ_max + y) * D, part);
    return;
  }
  w -= n_q;  // one row of T per workgroup
  const int nw = n_rep * ((NKB_max + 31) >> 5);
  int32_t* tail = T + static_cast<size_t>(w) * NKB_max + (NKB_max - nw);
  for (int i = threadIdx.x; i < nw; i += kMaskThreads) tail[i] = 0;
}

// ---------------------------------------------------------------- scores

// Workgroup (b*H_kv + g, y, z) computes the 64 x 64 tile of scores of the
// group's pooled Q-block rows 64z .. 64z+63 (row r = head r / nq, Q-block
// r % nq) against KV blocks 64y .. 64y+63 on the bf16 matrix cores, with each
// fp32 operand split in two bf16 parts: x = hi + lo, hi = bf16(x),
// lo = bf16(x - hi), so that |x - hi - lo| <= 2^-16 |x|.  A product is taken
// as hi*hi + hi*lo + lo*hi (three v_mfma_f32_32x32x16_bf16 per 16 dimensions;
// products of bf16 values are exact in fp32), which leaves out lo*lo and the
// two split residuals, each at most 2^-16 of |q_d k_d|: a score is within
// 3 * 2^-16 sum_d |q_d k_d| (plus fp32 accumulation) of the fp32 dot product.
// The split is made once, as the 64 x D fp32 tiles are staged into LDS as
// four bf16 tiles (rows padded by 16 bytes); wave w computes the 32 x 32
// block (KV blocks 32 (w / 2) .., Q rows 32 (w % 2) ..) as S^T = Kbar Qbar^T,
// lane l taking dimensions 8 (l / 32) .. + 7 of each 16-wide step of row
// l % 32 of both operands.  Its 16 results are KV blocks 8(r/4) + 4(l/32) +
// r%4 of Q row l % 32: four 16-byte stores (when rows of the score matrix are
// 16-byte aligned; else single floats).
constexpr int kScoreTile = 64;

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// hi and lo bf16 parts of four fp32 values
__device__ __forceinline__ void split_bf16x4(const float4 x, uint2& hi, uint2& lo) {
  const float v[4] = {x.x, x.y, x.z, x.w};
  __bf16 h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = static_cast<__bf16>(v[i]);
    l[i] = static_cast<__bf16>(v[i] - static_cast<float>(h[i]));
  }
  hi = make_uint2(__builtin_bit_cast(uint16_t, h[0]) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h[1])) << 16),
                  __builtin_bit_cast(uint16_t, h[2]) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h[3])) << 16));
  lo = make_uint2(__builtin_bit_cast(uint16_t, l[0]) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l[1])) << 16),
                  __builtin_bit_cast(uint16_t, l[2]) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l[3])) << 16));
}

template <int D>
__global__ __launch_bounds__(kMaskThreads) void block_scores_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int H_q, int H_kv,
    int NQ_max, int NKB_max, SeqInfo seq, float* __restrict__ scores, SelLens dl) {
  constexpr int RB = 2 * D + 16;  // padded row stride of a bf16 tile (bytes)
  __shared__ __attribute__((aligned(16))) char Qh[kScoreTile * RB];
  __shared__ __attribute__((aligned(16))) char Ql[kScoreTile * RB];
  __shared__ __attribute__((aligned(16))) char Kh[kScoreTile * RB];
  __shared__ __attribute__((aligned(16))) char Kl[kScoreTile * RB];
  const int bg = blockIdx.x;
  const int b = bg / H_kv;
  const int g = bg - b * H_kv;
  const int G = H_q / H_kv;
  int P, C;
  sel_lengths(dl, seq, b, P, C);
  const int pblk = P / 64;
  const int nq = C / 64;
  const int kb0 = static_cast<int>(blockIdx.y) * kScoreTile;
  const int r0 = static_cast<int>(blockIdx.z) * kScoreTile;
  const int n_rows = G * nq;
  if (kb0 >= pblk || r0 >= n_rows) return;
  const int tid = threadIdx.x;
  const size_t head_row0 = (static_cast<size_t>(b) * H_q + g * G) * NQ_max;
  auto row_index = [&](int r) {
    const int hl = r / nq;
    return head_row0 + static_cast<size_t>(hl) * NQ_max + (r - hl * nq);
  };
  // stage both tiles: D / 4 float4 per row, rows past the range as zeros; all
  // loads in flight before the split and the LDS writes
  constexpr int F4 = kScoreTile * D / 4 / kMaskThreads;  // float4 per thread per tile
  float4 qv[F4], kv[F4];
#pragma unroll
  for (int i = 0; i < F4; ++i) {
    const int e = tid + i * kMaskThreads;  // float4 index in the tile
    const int row = e / (D / 4), c4 = e - row * (D / 4);
    const int r = r0 + row, kb = kb0 + row;
    qv[i] = r < n_rows ? reinterpret_cast<const float4*>(qbar + row_index(r) * D)[c4]
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    kv[i] = kb < pblk
                ? reinterpret_cast<const float4*>(kbar + (static_cast<size_t>(bg) * NKB_max + kb) * D)[c4]
                : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < F4; ++i) {
    const int e = tid + i * kMaskThreads;
    const int row = e / (D / 4), c4 = e - row * (D / 4);
    const int off = row * RB + 8 * c4;
    uint2 hi, lo;
    split_bf16x4(qv[i], hi, lo);
    *reinterpret_cast<uint2*>(&Qh[off]) = hi;
    *reinterpret_cast<uint2*>(&Ql[off]) = lo;
    split_bf16x4(kv[i], hi, lo);
    *reinterpret_cast<uint2*>(&Kh[off]) = hi;
    *reinterpret_cast<uint2*>(&Kl[off]) = lo;
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int kb_blk = 32 * (wave >> 1), q_blk = 32 * (wave & 1);
  const int ka = (kb_blk + l32) * RB + 16 * hh;
  const int qa = (q_blk + l32) * RB + 16 * hh;
  f32x16_t acc = {};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {  // dimensions 16 s + 8 hh .. + 7 of this lane
    const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(&Kh[ka + 32 * s]);
    const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(&Kl[ka + 32 * s]);
    const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(&Qh[qa + 32 * s]);
    const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(&Ql[qa + 32 * s]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc, 0, 0, 0);
  }
  const int r = r0 + q_blk + l32;
  if (r >= n_rows) return;
  float* dst = scores + row_index(r) * NKB_max;
  const bool vec = (NKB_max & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kb = kb0 + kb_blk + 8 * j + 4 * hh;  // results 4j .. 4j+3: four consecutive blocks
    if (vec && kb + 3 < pblk) {
      *reinterpret_cast<float4*>(dst + kb) =
          make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (kb + k < pblk) dst[kb + k] = acc[4 * j + k];
    }
  }
}

// ---------------------------------------------------------------- selection

// Order-preserving map of a float to an unsigned key (-0 taken as +0).
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup per mask row (b, h, qb).  The budget-th largest candidate key
// is found by a most-significant-digit-first radix select (up to four 8-bit
// passes over the row, histograms in LDS).  When the digit bin that holds it
// is taken whole (the usual case once the bin is one key), the select stops
// and every thread decides its blocks alone; otherwise (equal keys straddle
// the budget) the row is written in ascending kb, taking keys above the
// threshold and, of the keys equal to it, the lowest kb first.
//
// kUnion: the fused selection also ORs each selected cell into its group's
// union bitmap at the tail of the T[b,g] row (cleared by select_pool_kernel).
// The row's bits are gathered in an LDS bitmap and ORed into the group's
// bitmap once, one device-scope atomicOr per nonzero word (rows that do not
// stage their keys in LDS, and rows with ties at the budget: per wave, one
// ballot over 64 consecutive blocks and up to two atomics).  The 128 rows of a
// group would all hit the same words, and atomics on one address serialize,
// so row r ORs into copy r % n_rep of the bitmap (n_rep copies side by side;
// the compaction ORs them together).  What is ORed is exactly the union over
// the chunk's Q-blocks and the group's heads (rows past the chunk select
// nothing).
// kLds: the row's candidate keys are read from the scores once (kTopkStage
// loads in flight per thread) into dynamic LDS (NKB_max words), and every pass
// reads them there; without it each pass re-reads the scores row.
// Where no tie straddles the budget, a thread decides four consecutive blocks
// at a time and writes their mask bytes as one 32-bit store.
template <bool kUnion, bool kLds>
__global__ __launch_bounds__(kMaskThreads) void topk_mask_kernel(
    const float* __restrict__ scores, int H_q, int NQ_max, int NKB_max, SeqInfo seq,
    int budget, int local, uint8_t* __restrict__ mask, int H_kv, int32_t* __restrict__ T,
    int n_rep, SelLens dl) {
  extern __shared__ uint32_t keys[];  // kLds: NKB_max keys; then (kUnion) the row's bitmap
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix, sh_need, sh_bin;
  __shared__ int wave_eq[kMaskThreads / 64];
  const size_t row = blockIdx.x;
  const int b = static_cast<int>(row / (static_cast<size_t>(H_q) * NQ_max));
  const int qb = static_cast<int>(row % NQ_max);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint8_t* mrow = mask + row * NKB_max;
  int P, C;
  sel_lengths(dl, seq, b, P, C);
  const int pblk = P / 64;
  const int nq = C / 64;
  // union bitmap of this row's group (kUnion): words at the tail of T[b,g]
  const int nwords = (NKB_max + 31) >> 5;
  uint32_t* ubits = nullptr;
  if (kUnion) {
    const int h = static_cast<int>((row / NQ_max) % H_q);
    const int g = h / (H_q / H_kv);
    ubits = reinterpret_cast<uint32_t*>(T + (static_cast<size_t>(b) * H_kv + g) * NKB_max +
                                        (NKB_max - n_rep * nwords) +
                                        static_cast<size_t>(row % n_rep) * nwords);
  }
  // OR the selections of blocks base + 64 * wave .. + 63 into the bitmap
  auto or_bits = [&](int base, bool sel) {
    const uint64_t bal = __ballot(sel);
    if (lane == 0 && bal != 0ull) {
      const int w0 = (base + 64 * wave) >> 5;
      const uint32_t lo = static_cast<uint32_t>(bal), hi = static_cast<uint32_t>(bal >> 32);
      if (lo != 0u && w0 < nwords) atomicOr(&ubits[w0], lo);
      if (hi != 0u && w0 + 1 < nwords) atomicOr(&ubits[w0 + 1], hi);
    }
  };
  // mask bytes of four consecutive blocks as one 32-bit store when the row allows
  const bool store4 = (NKB_max & 3) == 0 && (reinterpret_cast<uintptr_t>(mrow) & 3) == 0;
  if (qb >= nq) {
    if (store4) {
      for (int kb = 4 * tid; kb < NKB_max; kb += 4 * kMaskThreads)
        *reinterpret_cast<uint32_t*>(mrow + kb) = 0u;
    } else {
      for (int kb = tid; kb < NKB_max; kb += kMaskThreads) mrow[kb] = 0;
    }
    return;
  }
  // the row's union bits, gathered in LDS (after the keys) and ORed into the
  // group's bitmap once; rows too long to stage their keys OR per wave instead
  constexpr bool kLdsBits = kUnion && kLds;
  uint32_t* lbits = keys + NKB_max;
  if (kLdsBits) {
    for (int i = tid; i < nwords; i += kMaskThreads) lbits[i] = 0u;
    __syncthreads();
  }
  const int lo_local = pblk - local > 1 ? pblk - local : 1;  // candidates: [1, lo_local)
  const int n_cand = lo_local - 1 > 0 ? lo_local - 1 : 0;
  const uint32_t kk = static_cast<uint32_t>(budget < n_cand ? budget : n_cand);
  const float* srow = scores + row * NKB_max;
  if (kLds && kk > 0u) {  // kk is uniform; candidates are [1, lo_local), lo_local >= 2
    for (int base = 1; base < lo_local; base += kMaskThreads * kTopkStage) {
      float v[kTopkStage];
#pragma unroll
      for (int j = 0; j < kTopkStage; ++j) {  // clamped, so no load waits on a branch
        const int kb = base + j * kMaskThreads + tid;
        v[j] = srow[kb < lo_local ? kb : lo_local - 1];
      }
#pragma unroll
      for (int j = 0; j < kTopkStage; ++j) {
        const int kb = base + j * kMaskThreads + tid;
        if (kb < lo_local) keys[kb] = score_key(v[j]);
      }
    }
    __syncthreads();
  }
  auto key_at = [&](int kb) -> uint32_t { return kLds ? keys[kb] : score_key(srow[kb]); };

  uint32_t prefix = 0u, need = kk;
  uint32_t lvl_mask = 0u;  // key bits the passes have fixed
  bool whole_bin = true;   // every candidate in prefix's bin is taken
  if (kk > 0u) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
      hist[tid] = 0u;
      __syncthreads();
      for (int kb = 1 + tid; kb < lo_local; kb += kMaskThreads) {
        const uint32_t key = key_at(kb);
        if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // wave 0 finds the digit holding the need-th largest key: lane l owns
        // digits 255-4l .. 252-4l; a scan over lanes gives the count above
        // each lane's digits, and the lane whose range covers `need` walks them
        uint32_t h[4], tot = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h[j] = hist[255 - 4 * lane - j];
          tot += h[j];
        }
        uint32_t inc = tot;
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = __shfl_up(inc, o);
          if (lane >= o) inc += y;
        }
        const uint32_t excl = inc - tot;
        const uint64_t hit = __ballot(excl < need && need <= inc);
        if (lane == __ffsll(static_cast<unsigned long long>(hit)) - 1) {
          uint32_t cum = excl;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (cum + h[j] >= need) {
              sh_prefix = prefix | (static_cast<uint32_t>(255 - 4 * lane - j) << shift);
              sh_need = need - cum;
              sh_bin = h[j];
              break;
            }
            cum += h[j];
          }
        }
      }
      __syncthreads();
      prefix = sh_prefix;
      need = sh_need;
      lvl_mask = 0xFFFFFFFFu << shift;
      whole_bin = need == sh_bin;
      // the digit's bin is taken whole: the budget is exactly the candidates
      // whose fixed bits are at least prefix, and the lower bits need no pass
      if (whole_bin) break;
    }
  }
  // prefix = the fixed bits of the budget-th largest candidate's key; take the
  // candidates above it, and `need` of those equal to it (lowest kb first)

  if (whole_bin && !(kUnion && !kLds)) {  // no equal key is left out: no ordering across the row
    // each thread decides four consecutive blocks per step
    for (int kb0 = 4 * tid; kb0 < NKB_max; kb0 += 4 * kMaskThreads) {
      uint32_t bytes = 0u, bits = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = kb0 + j;
        bool sel = (pblk > 0 && kb == 0) || (kb >= lo_local && kb < pblk) ||
                   (kb >= pblk && kb <= pblk + qb);
        if (kk > 0u && kb >= 1 && kb < lo_local)
          sel = sel || (key_at(kb) & lvl_mask) >= prefix;
        sel = sel && kb < NKB_max;
        bytes |= static_cast<uint32_t>(sel) << (8 * j);
        bits |= static_cast<uint32_t>(sel) << j;
      }
      if (store4) {
        *reinterpret_cast<uint32_t*>(mrow + kb0) = bytes;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (kb0 + j < NKB_max) mrow[kb0 + j] = static_cast<uint8_t>(bytes >> (8 * j));
      }
      if (kLdsBits && bits != 0u) atomicOr(&lbits[kb0 >> 5], bits << (kb0 & 31));
    }
    if (kLdsBits) {
      __syncthreads();
      for (int i = tid; i < nwords; i += kMaskThreads)
        if (lbits[i] != 0u) atomicOr(&ubits[i], lbits[i]);
    }
    return;
  }
  if (whole_bin) {  // rows too long for LDS: one block per thread, ORs per wave
    for (int base = 0; base < NKB_max; base += kMaskThreads) {
      const int kb = base + tid;
      bool sel = false;
      if (kb < NKB_max) {
        sel = (pblk > 0 && kb == 0) || (kb >= lo_local && kb < pblk) ||
              (kb >= pblk && kb <= pblk + qb);
        if (kk > 0u && kb >= 1 && kb < lo_local)
          sel = sel || (key_at(kb) & lvl_mask) >= prefix;
        mrow[kb] = sel ? 1 : 0;
      }
      or_bits(base, sel);
    }
    return;
  }

  uint32_t taken = 0u;  // equals already taken (uniform)
  for (int base = 0; base < NKB_max; base += kMaskThreads) {
    const int kb = base + tid;
    bool sel = false, eq = false;
    if (kb < NKB_max) {
      sel = (pblk > 0 && kb == 0) || (kb >= lo_local && kb < pblk) ||
            (kb >= pblk && kb <= pblk + qb);
      if (kk > 0u && kb >= 1 && kb < lo_local) {
        const uint32_t key = key_at(kb);
        sel = sel || key > prefix;
        eq = key == prefix;
      }
    }
    const uint64_t bal = __ballot(eq);
    const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
    if (lane == 0) wave_eq[wave] = __popcll(bal);
    __syncthreads();
    uint32_t off = taken;
    for (int w = 0; w < wave; ++w) off += wave_eq[w];
    if (eq && off + below < need) sel = true;
    if (kb < NKB_max) mrow[kb] = sel ? 1 : 0;
    if (kUnion) or_bits(base, sel);
    for (int w = 0; w < kMaskThreads / 64; ++w) taken += wave_eq[w];
    __syncthreads();
  }
}

template <bool kUnion>
void launch_topk(const float* scores, int B, int H_q, int NQ_max, int NKB_max, const SeqInfo& seq,
                 int budget, int local, uint8_t* mask, int H_kv, int32_t* T, int n_rep,
                 const SelLens& dl, hipStream_t stream) {
  const dim3 grid(B * H_q * NQ_max);
  const size_t bitmap = kUnion ? static_cast<size_t>((NKB_max + 31) / 32) * sizeof(uint32_t) : 0;
  if (NKB_max <= kTopkLdsMax)  // keys, then the row's union bits
    hipLaunchKernelGGL((topk_mask_kernel<kUnion, true>), grid, dim3(kMaskThreads),
                       static_cast<size_t>(NKB_max) * sizeof(uint32_t) + bitmap, stream, scores,
                       H_q, NQ_max, NKB_max, seq, budget, local, mask, H_kv, T, n_rep, dl);
  else
    hipLaunchKernelGGL((topk_mask_kernel<kUnion, false>), grid, dim3(kMaskThreads), 0, stream,
                       scores, H_q, NQ_max, NKB_max, seq, budget, local, mask, H_kv, T, n_rep,
                       dl);
}

}  // namespace

hipError_t launch_pool_blocks(const void* X, int esz, int B, int H, int64_t R, int D,
                              const BlockRange& rng, int max_span, float* out, int NB_out,
                              hipStream_t stream) {
  if (max_span <= 0) return hipSuccess;
  const dim3 grid(B * H, max_span);
  if (esz == 2) {
    const __bf16* x = static_cast<const __bf16*>(X);
    if (D == 128)
      hipLaunchKernelGGL((pool_blocks_kernel<__bf16, 128>), grid, dim3(kMaskThreads), 0, stream,
                         x, H, R, rng, out, NB_out);
    else
      hipLaunchKernelGGL((pool_blocks_kernel<__bf16, 64>), grid, dim3(kMaskThreads), 0, stream,
                         x, H, R, rng, out, NB_out);
  } else {
    const float* x = static_cast<const float*>(X);
    if (D == 128)
      hipLaunchKernelGGL((pool_blocks_kernel<float, 128>), grid, dim3(kMaskThreads), 0, stream,
                         x, H, R, rng, out, NB_out);
    else
      hipLaunchKernelGGL((pool_blocks_kernel<float, 64>), grid, dim3(kMaskThreads), 0, stream, x,
                         H, R, rng, out, NB_out);
  }
  return hipGetLastError();
}

namespace {

hipError_t launch_scores(const float* qbar, const float* kbar, int B, int H_q, int H_kv,
                         int NQ_max, int NKB_max, int D, const SeqInfo& seq, int max_pblk,
                         float* scores, const SelLens& dl, hipStream_t stream) {
  if (max_pblk <= 0) return hipSuccess;
  const int ny = (max_pblk + kScoreTile - 1) / kScoreTile;
  const int nz = ((H_q / H_kv) * NQ_max + kScoreTile - 1) / kScoreTile;
  const dim3 grid(B * H_kv, ny, nz);
  if (D == 128)
    hipLaunchKernelGGL(block_scores_kernel<128>, grid, dim3(kMaskThreads), 0, stream, qbar, kbar,
                       H_q, H_kv, NQ_max, NKB_max, seq, scores, dl);
  else
    hipLaunchKernelGGL(block_scores_kernel<64>, grid, dim3(kMaskThreads), 0, stream, qbar, kbar,
                       H_q, H_kv, NQ_max, NKB_max, seq, scores, dl);
  return hipGetLastError();
}

template <typename TIn>
void launch_select_pool(const void* Q, const void* K, int B, int H_q, int H_kv, int C_max,
                        int64_t L, int D, const SeqInfo& seq, int span, float* qbar, int NQ_max,
                        float* kbar, int NKB_max, int32_t* T, int n_rep, const AppendSrc* app,
                        const SelLens& dl, hipStream_t stream) {
  const int n_k = B * H_kv * span, n_q = B * H_q * span;
  const dim3 grid((app ? 2 * n_k : n_k) + n_q + B * H_kv);
  const TIn* k = static_cast<const TIn*>(K);
  const TIn* q = static_cast<const TIn*>(Q);
  if (app) {
    const TIn* kn = static_cast<const TIn*>(app->k_new);
    const TIn* vn = static_cast<const TIn*>(app->v_new);
    TIn* kc = static_cast<TIn*>(app->k_cache);
    TIn* vc = static_cast<TIn*>(app->v_cache);
    if (D == 128)
      hipLaunchKernelGGL((select_pool_kernel<TIn, 128, true>), grid, dim3(kMaskThreads), 0,
                         stream, nullptr, q, H_q, H_kv, L, C_max, NQ_max, NKB_max, span, n_k, n_q,
                         n_rep, seq, kbar, qbar, T, kn, vn, kc, vc, dl);
    else
      hipLaunchKernelGGL((select_pool_kernel<TIn, 64, true>), grid, dim3(kMaskThreads), 0,
                         stream, nullptr, q, H_q, H_kv, L, C_max, NQ_max, NKB_max, span, n_k, n_q,
                         n_rep, seq, kbar, qbar, T, kn, vn, kc, vc, dl);
    return;
  }
  if (D == 128)
    hipLaunchKernelGGL((select_pool_kernel<TIn, 128, false>), grid, dim3(kMaskThreads), 0, stream,
                       k, q, H_q, H_kv, L, C_max, NQ_max, NKB_max, span, n_k, n_q, n_rep, seq,
                       kbar, qbar, T, nullptr, nullptr, nullptr, nullptr, dl);
  else
    hipLaunchKernelGGL((select_pool_kernel<TIn, 64, false>), grid, dim3(kMaskThreads), 0, stream,
                       k, q, H_q, H_kv, L, C_max, NQ_max, NKB_max, span, n_k, n_q, n_rep, seq,
                       kbar, qbar, T, nullptr, nullptr, nullptr, nullptr, dl);
}

}  // namespace

hipError_t launch_block_mask(const float* qbar, const float* kbar, int B, int H_q, int H_kv,
                             int NQ_max, int NKB_max, int D, const SeqInfo& seq, int max_pblk,
                             int budget, int local, float* scores, uint8_t* mask,
                             hipStream_t stream) {
  const SelLens host{};  // host lengths
  const hipError_t e = launch_scores(qbar, kbar, B, H_q, H_kv, NQ_max, NKB_max, D, seq, max_pblk,
                                     scores, host, stream);
  if (e != hipSuccess) return e;
  launch_topk<false>(scores, B, H_q, NQ_max, NKB_max, seq, budget, local, mask, H_kv, nullptr, 1,
                     host, stream);
  return hipGetLastError();
}

hipError_t launch_select_chunk(const void* Q, const void* K, int esz, int B, int H_q, int H_kv,
                               int C_max, int64_t L, int D, const SeqInfo& seq, int max_nq,
                               int max_pblk, int budget, int local, float* qbar, int NQ_max,
                               float* kbar, int NKB_max, float* scores, uint8_t* mask,
                               int32_t* T, int32_t* len, const AppendSrc* app, const SelLens& dl,
                               hipStream_t stream) {
  // copies of the union bitmap the top-k rows spread their atomics over (as many
  // as the T row's tail holds, up to 16)
  const int nwords = (NKB_max + 31) / 32;
  const int n_rep = std::max(1, std::min(kSelectReplicas, NKB_max / nwords));
  if (esz == 2)
    launch_select_pool<__bf16>(Q, K, B, H_q, H_kv, C_max, L, D, seq, max_nq, qbar, NQ_max, kbar,
                               NKB_max, T, n_rep, app, dl, stream);
  else
    launch_select_pool<float>(Q, K, B, H_q, H_kv, C_max, L, D, seq, max_nq, qbar, NQ_max, kbar,
                              NKB_max, T, n_rep, app, dl, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_scores(qbar, kbar, B, H_q, H_kv, NQ_max, NKB_max, D, seq, max_pblk, scores, dl,
                    stream);
  if (e != hipSuccess) return e;
  launch_topk<true>(scores, B, H_q, NQ_max, NKB_max, seq, budget, local, mask, H_kv, T, n_rep,
                    dl, stream);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_union_compact(B * H_kv, NKB_max, n_rep, T, len, stream);
}

}  // namespace ca
