// A lightweight block-mask producer on gfx950 (the step upstream of the
// union).  CompactAttention, "Methodology" (selection stage) and the problem
// statement of the technical summaries: the union takes a per-head 2D block
// mask from any lightweight pattern search, and that search runs again over
// the growing KV cache at every chunk, so its cost matters.  The pages leave
// the searcher open; this one is training-free:
//
//   qbar[b,h,qb]  = mean of the 64 rows of Q-block qb          (pool_blocks)
//   kbar[b,g,kb]  = mean of the 64 rows of KV block kb         (pool_blocks,
//                   kept across chunks: only the new blocks are pooled)
//   s[b,h,qb,kb]  = qbar . kbar                                (block_scores,
//                   fp32 on the matrix cores)
//   mask row      = sink + last `local` prior blocks + causal block triangle
//                   + the `budget` best remaining prior blocks  (topk_mask)
//
// All three are HBM/L2-bound and tiny next to the attention: pooling reads
// each new block once; the scores read kbar once per KV group; the selection
// reads each score row a few times from L2 and writes one mask byte per cell.

#include "kernels.hpp"

namespace ca {
namespace {

constexpr int kMaskThreads = 256;

// ---------------------------------------------------------------- pooling

// Workgroup (b*H + h, y) pools block kb = begin[b] + y.  Each thread sums a
// 16-byte column slice over every RPI-th row of the block; the RPI partial
// sums of a column are then added in row-group order.
template <typename TIn, int D>
__global__ __launch_bounds__(kMaskThreads) void pool_blocks_kernel(const TIn* __restrict__ X,
                                                                   int H, int64_t R,
                                                                   BlockRange rng,
                                                                   float* __restrict__ out,
                                                                   int NB_out) {
  constexpr int V = 16 / static_cast<int>(sizeof(TIn));  // elements per 16-byte load
  constexpr int TPR = D / V;                              // threads per row
  constexpr int RPI = kMaskThreads / TPR;                 // rows per iteration
  static_assert(64 % RPI == 0, "rows of a block split evenly over the row groups");
  __shared__ float part[RPI * D];
  const int bh = blockIdx.x;
  const int b = bh / H;
  const int kb = rng.begin[b] + static_cast<int>(blockIdx.y);
  if (kb >= rng.end[b]) return;
  const int tid = threadIdx.x;
  const int col = (tid % TPR) * V;
  const int rsub = tid / TPR;
  const TIn* src = X + (static_cast<size_t>(bh) * R + static_cast<size_t>(kb) * 64) * D + col;
  // all of this thread's row loads in flight before the sums (in row order)
  constexpr int NR = 64 / RPI;
  uint4 raw[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k)
    raw[k] = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(rsub + k * RPI) * D);
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const TIn* e = reinterpret_cast<const TIn*>(&raw[k]);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += static_cast<float>(e[i]);
  }
#pragma unroll
  for (int i = 0; i < V; ++i) part[rsub * D + col + i] = acc[i];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int k = 0; k < RPI; ++k) s += part[k * D + tid];
    out[(static_cast<size_t>(bh) * NB_out + kb) * D + tid] = s * (1.f / 64.f);
  }
}

// ---------------------------------------------------------------- scores

// Workgroup (b*H_kv + g, y, z) computes the 64 x 64 tile of scores of the
// group's pooled Q-block rows 64z .. 64z+63 (row r = head r / nq, Q-block
// r % nq) against KV blocks 64y .. 64y+63, on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32, twice the fp32 rate of the vector ALUs with packed
// fp32 off).  Both 64 x D operand tiles are staged in LDS whole (rows padded
// by 16 bytes, so the 32 rows a read touches fall in distinct banks); wave w
// computes the 32 x 32 block (KV blocks 32 (w / 2) .., Q rows 32 (w % 2) ..)
// as S^T = Kbar Qbar^T over D/2 steps of 2 dimensions.  Lane l takes the
// dimensions (l / 32) * D/2 + s of step s, so its operands for four steps are
// one 16-byte read.  Its 16 results are KV blocks 8(r/4) + 4(l/32) + r%4 of
// Q row l % 32: four 16-byte stores (when rows of the score matrix are
// 16-byte aligned; else single floats).
constexpr int kScoreTile = 64;

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int D>
__global__ __launch_bounds__(kMaskThreads) void block_scores_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int H_q, int H_kv,
    int NQ_max, int NKB_max, SeqInfo seq, float* __restrict__ scores) {
  constexpr int RS = D + 4;  // padded row stride (floats)
  __shared__ __attribute__((aligned(16))) float Qs[kScoreTile * RS];
  __shared__ __attribute__((aligned(16))) float Ks[kScoreTile * RS];
  const int bg = blockIdx.x;
  const int b = bg / H_kv;
  const int g = bg - b * H_kv;
  const int G = H_q / H_kv;
  const int pblk = seq.prior[b] / 64;
  const int nq = seq.chunk[b] / 64;
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
  // loads in flight before the LDS writes
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
    *reinterpret_cast<float4*>(&Qs[row * RS + 4 * c4]) = qv[i];
    *reinterpret_cast<float4*>(&Ks[row * RS + 4 * c4]) = kv[i];
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int kb_blk = 32 * (wave >> 1), q_blk = 32 * (wave & 1);
  const float* ka = &Ks[(kb_blk + l32) * RS + hh * (D / 2)];
  const float* qa = &Qs[(q_blk + l32) * RS + hh * (D / 2)];
  f32x16_t acc = {};
#pragma unroll
  for (int s = 0; s < D / 2; s += 4) {
    const float4 a4 = *reinterpret_cast<const float4*>(ka + s);
    const float4 b4 = *reinterpret_cast<const float4*>(qa + s);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.x, b4.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.y, b4.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.z, b4.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.w, b4.w, acc, 0, 0, 0);
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
__global__ __launch_bounds__(kMaskThreads) void topk_mask_kernel(
    const float* __restrict__ scores, int H_q, int NQ_max, int NKB_max, SeqInfo seq,
    int budget, int local, uint8_t* __restrict__ mask) {
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
  const int pblk = seq.prior[b] / 64;
  const int nq = seq.chunk[b] / 64;
  if (qb >= nq) {
    for (int kb = tid; kb < NKB_max; kb += kMaskThreads) mrow[kb] = 0;
    return;
  }
  const int lo_local = pblk - local > 1 ? pblk - local : 1;  // candidates: [1, lo_local)
  const int n_cand = lo_local - 1 > 0 ? lo_local - 1 : 0;
  const uint32_t kk = static_cast<uint32_t>(budget < n_cand ? budget : n_cand);
  const float* srow = scores + row * NKB_max;

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
        const uint32_t key = score_key(srow[kb]);
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

  if (whole_bin) {  // no equal key is left out: no ordering across the row
    for (int kb = tid; kb < NKB_max; kb += kMaskThreads) {
      bool sel = (pblk > 0 && kb == 0) || (kb >= lo_local && kb < pblk) ||
                 (kb >= pblk && kb <= pblk + qb);
      if (kk > 0u && kb >= 1 && kb < lo_local) sel = sel || (score_key(srow[kb]) & lvl_mask) >= prefix;
      mrow[kb] = sel ? 1 : 0;
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
        const uint32_t key = score_key(srow[kb]);
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
    for (int w = 0; w < kMaskThreads / 64; ++w) taken += wave_eq[w];
    __syncthreads();
  }
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

hipError_t launch_block_mask(const float* qbar, const float* kbar, int B, int H_q, int H_kv,
                             int NQ_max, int NKB_max, int D, const SeqInfo& seq, int max_pblk,
                             int budget, int local, float* scores, uint8_t* mask,
                             hipStream_t stream) {
  if (max_pblk > 0) {
    const int ny = (max_pblk + kScoreTile - 1) / kScoreTile;
    const int nz = ((H_q / H_kv) * NQ_max + kScoreTile - 1) / kScoreTile;
    const dim3 grid(B * H_kv, ny, nz);
    if (D == 128)
      hipLaunchKernelGGL(block_scores_kernel<128>, grid, dim3(kMaskThreads), 0, stream, qbar,
                         kbar, H_q, H_kv, NQ_max, NKB_max, seq, scores);
    else
      hipLaunchKernelGGL(block_scores_kernel<64>, grid, dim3(kMaskThreads), 0, stream, qbar, kbar,
                         H_q, H_kv, NQ_max, NKB_max, seq, scores);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topk_mask_kernel, dim3(B * H_q * NQ_max), dim3(kMaskThreads), 0, stream,
                     scores, H_q, NQ_max, NKB_max, seq, budget, local, mask);
  return hipGetLastError();
}

}  // namespace ca
