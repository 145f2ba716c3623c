// Zero-copy paged chunk attention, fp32 on the vector ALUs.
//
// Same contract as the bf16 path (CompactAttention, execution stage: the
// block table drives a paged dense attention that reads the selected blocks
// in place from the KV-head-major cache), for fp32 inputs, where fp32
// arithmetic is kept end to end.  It serves small chunks, where latency
// rather than arithmetic sets the time.  A workgroup of 512 threads owns 64
// consecutive query rows of one head, eight threads per row (32 rows, sixteen
// threads per row, when 64-row tiles would leave most CUs idle), each thread
// holding its share of the row's q and output accumulator; a score is the sum
// of the partial dot products (DPP lane moves, fused into the adds).  Each selected block's K
// and V rows are staged in LDS (coalesced 16-byte loads) and read back as
// broadcasts.  With per-(head, Q-block) tables (the lists of a block-sparse
// kernel) the workgroup's rows lie inside one Q-block, so it simply reads that
// Q-block's table row.

#include "kernels.hpp"

namespace ca {
namespace {

constexpr int kBlk = 64;
constexpr int kThreadsF = 512;  // threads per workgroup

// Sum over the R lanes of a row (R = 8 or 16 consecutive lanes, aligned), in
// every one of them, by DPP moves on the vector ALU (no LDS round trip): swap
// neighbours, swap pairs, add the mirror image within 8 lanes, then within 16.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, true));
}
template <int R>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(R == 8 || R == 16, "row width");
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp<0x141>(x);  // row_half_mirror: lane 7 - i within each 8 lanes
  if (R == 16) x += dpp<0x140>(x);  // row_mirror: lane 15 - i within each 16 lanes
  return x;
}

// kTpr threads per query row (8, or 16 when 64-row tiles would leave most CUs
// idle: twice the workgroups, each thread with half the products); a
// workgroup owns kThreadsF / kTpr consecutive rows.  kSplit: the table is cut
// into p.n_split contiguous position ranges, one per workgroup, and each
// writes its unnormalised output, running max and denominator to part_o /
// part_ml for the split-KV merge (more workgroups for small chunks).
template <int D, int kTpr, bool kSplit>
__global__ __launch_bounds__(kThreadsF) void chunk_attn_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const int32_t* __restrict__ T, const int32_t* __restrict__ len, float* __restrict__ O,
    float* __restrict__ lse, AttnParams p, SeqInfo seq, int n_tiles, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int kRowsF = kThreadsF / kTpr;
  constexpr int SL = D / kTpr;  // this thread's slice of the row
  __shared__ __attribute__((aligned(16))) float Ks[kBlk * D];
  __shared__ __attribute__((aligned(16))) float Vs[kBlk * D];

  const int tid = threadIdx.x;
  const int wg = blockIdx.x;
  const int nsp = kSplit ? p.n_split : 1;
  const int bhs = wg / n_tiles;  // (head, split)
  const int tile = wg - bhs * n_tiles;
  const int bh = bhs / nsp;
  const int split = bhs - bh * nsp;
  const int rank = bh / p.H_q;
  const int h = bh - rank * p.H_q;
  const int b = seq.order[rank];
  const int g = h / p.G;
  int P, C;
  seq_lengths(p, seq, b, P, C);
  const int bg = b * p.H_kv + g;

  const int row = tile * kRowsF + tid / kTpr;
  const int part = tid % kTpr;
  const bool row_in = row < p.C_max;
  const bool row_live = row < C;
  const size_t qrow = (static_cast<size_t>(b) * p.H_q + h) * p.C_max + row;
  const size_t qo = qrow * D + part * SL;

  if (tile * kRowsF >= C) {  // padding rows only (the merge writes them when split)
    if (row_in && !kSplit) {
      for (int i = 0; i < SL; ++i) O[qo + i] = 0.f;
      if (lse && part == 0) lse[qrow] = -INFINITY;
    }
    return;
  }
  const int last_row = min(C, (tile + 1) * kRowsF) - 1;
  const int kb_limit = (P + last_row) / kBlk;
  const int nkb = (P + C + kBlk - 1) / kBlk;
  // table of the workgroup: T[b,g], or T[b,h,Q-block] for per-Q-block lists
  const size_t trow = p.row_tables ? (static_cast<size_t>(b) * p.H_q + h) * p.NQ_max +
                                         (tile * kRowsF) / kBlk
                                   : static_cast<size_t>(bg);
  int nT = len[trow];
  nT = nT < 0 ? 0 : (nT > p.NKB_max ? p.NKB_max : nT);
  const int32_t* Trow = T + trow * p.NKB_max;
  const size_t kv_base = static_cast<size_t>(bg) * static_cast<size_t>(p.L) * D;

  float q[SL], acc[SL];
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    q[i] = row_in ? Q[qo + i] : 0.f;
    acc[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int qpos = P + row;

  // The next listed block's K and V are loaded into registers while the
  // current one is computed, then stored to LDS at the top of the next step.
  constexpr int NV = kBlk * D / 4 / kThreadsF;  // 16-byte pieces per thread
  float4 pk[NV], pv[NV];
  auto valid = [&](int kb) { return kb >= 0 && kb < nkb && kb <= kb_limit; };
  // this workgroup's range of table positions: all of them without splitting
  const int lo = kSplit ? static_cast<int>((static_cast<int64_t>(nT) * split) / nsp) : 0;
  const int hi = kSplit ? static_cast<int>((static_cast<int64_t>(nT) * (split + 1)) / nsp) : nT;
  auto next_valid = [&](int jj) {
    while (jj < hi && !valid(Trow[jj])) ++jj;
    return jj;
  };
  auto kv_piece = [&](const float* base, int jj, int i) {
    const size_t off = kv_base + static_cast<size_t>(Trow[jj]) * kBlk * D;
    return reinterpret_cast<const float4*>(base + off)[tid + i * kThreadsF];
  };
  int jn = next_valid(lo);
  if (jn < hi) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      pk[i] = kv_piece(K, jn, i);
      pv[i] = kv_piece(V, jn, i);
    }
  }
  while (jn < hi) {
    const int kb = Trow[jn];
    __syncthreads();  // previous block fully consumed
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      reinterpret_cast<float4*>(Ks)[tid + i * kThreadsF] = pk[i];
      reinterpret_cast<float4*>(Vs)[tid + i * kThreadsF] = pv[i];
    }
    jn = next_valid(jn + 1);
    if (jn < hi) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        pk[i] = kv_piece(K, jn, i);
        pv[i] = kv_piece(V, jn, i);
      }
    }
    __syncthreads();

    float s[kBlk];  // fully unrolled loops keep the scores in registers
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kBlk; ++k) {
      const float* kr = Ks + k * D + part * SL;
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < SL; ++i) dot = __builtin_fmaf(q[i], kr[i], dot);
      float sc = row_sum<kTpr>(dot);
      if (kb * kBlk + k > qpos) sc = -INFINITY;
      s[k] = sc;
      mx = fmaxf(mx, sc);
    }
    if (mx == -INFINITY) continue;  // no admissible key of this block for this row
    const float m_new = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * p.scale_log2);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < SL; ++i) acc[i] *= alpha;
    m = m_new;
#pragma unroll
    for (int k = 0; k < kBlk; ++k) {
      const float w = __builtin_amdgcn_exp2f((s[k] - m) * p.scale_log2);
      l += w;
      const float* vr = Vs + k * D + part * SL;
#pragma unroll
      for (int i = 0; i < SL; ++i) acc[i] = __builtin_fmaf(w, vr[i], acc[i]);
    }
  }

  if (!row_in) return;
  if (kSplit) {  // partial results: acc (unnormalised), running max, denominator
    if (!row_live) return;
    const size_t prow = static_cast<size_t>(split) * p.rows_total + qrow;
    for (int i = 0; i < SL; ++i) part_o[prow * D + part * SL + i] = acc[i];
    if (part == 0) {
      part_ml[2 * prow] = m;
      part_ml[2 * prow + 1] = l;
    }
    return;
  }
  const float inv = (row_live && l > 0.f) ? 1.f / l : 0.f;
  for (int i = 0; i < SL; ++i) O[qo + i] = row_live ? acc[i] * inv : 0.f;
  if (lse && part == 0)
    lse[qrow] = (row_live && l > 0.f) ? m * p.scale + __logf(l) : -INFINITY;
}

template <bool kSplit>
hipError_t launch_f32(const float* Q, const float* K, const float* V, const int32_t* T,
                      const int32_t* len, float* O, float* lse, int B, int D,
                      const AttnParams& p, const SeqInfo& seq, float* part_o, float* part_ml,
                      hipStream_t stream) {
  // 16 threads per row (32-row tiles) when 64-row tiles would occupy fewer
  // workgroups than the device has CUs
  const int nsp = kSplit ? p.n_split : 1;
  const bool narrow = static_cast<int64_t>(B) * p.H_q * nsp * ((p.C_max + 63) / 64) < p.cus;
  const int rows = narrow ? kThreadsF / 16 : kThreadsF / 8;
  const int n_tiles = (p.C_max + rows - 1) / rows;
  const dim3 grid(B * p.H_q * nsp * n_tiles), block(kThreadsF);
  if (D == 128 && narrow)
    hipLaunchKernelGGL((chunk_attn_f32_kernel<128, 16, kSplit>), grid, block, 0, stream, Q, K, V,
                       T, len, O, lse, p, seq, n_tiles, part_o, part_ml);
  else if (D == 128)
    hipLaunchKernelGGL((chunk_attn_f32_kernel<128, 8, kSplit>), grid, block, 0, stream, Q, K, V,
                       T, len, O, lse, p, seq, n_tiles, part_o, part_ml);
  else if (narrow)
    hipLaunchKernelGGL((chunk_attn_f32_kernel<64, 16, kSplit>), grid, block, 0, stream, Q, K, V,
                       T, len, O, lse, p, seq, n_tiles, part_o, part_ml);
  else
    hipLaunchKernelGGL((chunk_attn_f32_kernel<64, 8, kSplit>), grid, block, 0, stream, Q, K, V,
                       T, len, O, lse, p, seq, n_tiles, part_o, part_ml);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_attn_f32(const float* Q, const float* K, const float* V,
                                 const int32_t* T, const int32_t* len, float* O, float* lse,
                                 int B, int D, const AttnParams& p, const SeqInfo& seq,
                                 hipStream_t stream) {
  return launch_f32<false>(Q, K, V, T, len, O, lse, B, D, p, seq, nullptr, nullptr, stream);
}

hipError_t launch_chunk_attn_f32_split(const float* Q, const float* K, const float* V,
                                       const int32_t* T, const int32_t* len, float* O,
                                       float* lse, int B, int D, const AttnParams& p,
                                       const SeqInfo& seq, float* part_o, float* part_ml,
                                       hipStream_t stream) {
  const hipError_t e =
      launch_f32<true>(Q, K, V, T, len, O, lse, B, D, p, seq, part_o, part_ml, stream);
  if (e != hipSuccess) return e;
  return launch_split_combine(part_o, part_ml, D, true, O, lse, p, seq, stream);
}

}  // namespace ca
