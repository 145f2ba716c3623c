// Zero-copy paged chunk attention, fp32 on the vector ALUs.
//
// Same contract as the bf16 path (CompactAttention, execution stage: the
// block table drives a paged dense attention that reads the selected blocks
// in place from the KV-head-major cache), for fp32 inputs, where fp32
// arithmetic is kept end to end.  It serves small chunks, where latency
// rather than arithmetic sets the time.  A workgroup of 512 threads owns 64
// consecutive query rows of one head, eight threads per row, each holding an
// eighth of the row's q and output accumulator; a score is the sum of the
// eight partial dot products (three lane exchanges).  Each selected block's K
// and V rows are staged in LDS (coalesced 16-byte loads) and read back as
// broadcasts.  With per-(head, Q-block) tables (the lists of a block-sparse
// kernel) the workgroup's 64 rows are exactly one Q-block, so it simply reads
// its own table row.

#include "kernels.hpp"

namespace ca {
namespace {

constexpr int kBlk = 64;
constexpr int kTpr = 8;  // threads per query row
constexpr int kRowsF = 64;
constexpr int kThreadsF = kRowsF * kTpr;

template <int D>
__global__ __launch_bounds__(kThreadsF) void chunk_attn_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const int32_t* __restrict__ T, const int32_t* __restrict__ len, float* __restrict__ O,
    float* __restrict__ lse, AttnParams p, SeqInfo seq, int n_tiles) {
  constexpr int SL = D / kTpr;  // this thread's slice of the row
  __shared__ __attribute__((aligned(16))) float Ks[kBlk * D];
  __shared__ __attribute__((aligned(16))) float Vs[kBlk * D];

  const int tid = threadIdx.x;
  const int wg = blockIdx.x;
  const int bh = wg / n_tiles;
  const int tile = wg - bh * n_tiles;
  const int rank = bh / p.H_q;
  const int h = bh - rank * p.H_q;
  const int b = seq.order[rank];
  const int g = h / p.G;
  const int P = seq.prior[b];
  const int C = seq.chunk[b];
  const int bg = b * p.H_kv + g;

  const int row = tile * kRowsF + tid / kTpr;
  const int part = tid % kTpr;
  const bool row_in = row < p.C_max;
  const bool row_live = row < C;
  const size_t qrow = (static_cast<size_t>(b) * p.H_q + h) * p.C_max + row;
  const size_t qo = qrow * D + part * SL;

  if (tile * kRowsF >= C) {  // padding rows only
    if (row_in) {
      for (int i = 0; i < SL; ++i) O[qo + i] = 0.f;
      if (lse && part == 0) lse[qrow] = -INFINITY;
    }
    return;
  }
  const int last_row = min(C, (tile + 1) * kRowsF) - 1;
  const int kb_limit = (P + last_row) / kBlk;
  const int nkb = (P + C + kBlk - 1) / kBlk;
  // table of the workgroup: T[b,g], or T[b,h,Q-block] for per-Q-block lists
  const size_t trow = p.row_tables ? (static_cast<size_t>(b) * p.H_q + h) * p.NQ_max + tile
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
  auto next_valid = [&](int jj) {
    while (jj < nT && !valid(Trow[jj])) ++jj;
    return jj;
  };
  auto kv_piece = [&](const float* base, int jj, int i) {
    const size_t off = kv_base + static_cast<size_t>(Trow[jj]) * kBlk * D;
    return reinterpret_cast<const float4*>(base + off)[tid + i * kThreadsF];
  };
  int jn = next_valid(0);
  if (jn < nT) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      pk[i] = kv_piece(K, jn, i);
      pv[i] = kv_piece(V, jn, i);
    }
  }
  while (jn < nT) {
    const int kb = Trow[jn];
    __syncthreads();  // previous block fully consumed
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      reinterpret_cast<float4*>(Ks)[tid + i * kThreadsF] = pk[i];
      reinterpret_cast<float4*>(Vs)[tid + i * kThreadsF] = pv[i];
    }
    jn = next_valid(jn + 1);
    if (jn < nT) {
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
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      float sc = dot + __shfl_xor(dot, 4);
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
  const float inv = (row_live && l > 0.f) ? 1.f / l : 0.f;
  for (int i = 0; i < SL; ++i) O[qo + i] = row_live ? acc[i] * inv : 0.f;
  if (lse && part == 0)
    lse[qrow] = (row_live && l > 0.f) ? m * p.scale + __logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_chunk_attn_f32(const float* Q, const float* K, const float* V,
                                 const int32_t* T, const int32_t* len, float* O, float* lse,
                                 int B, int D, const AttnParams& p, const SeqInfo& seq,
                                 hipStream_t stream) {
  const int n_tiles = (p.C_max + kRowsF - 1) / kRowsF;
  const dim3 grid(B * p.H_q * n_tiles), block(kThreadsF);
  if (D == 128)
    hipLaunchKernelGGL(chunk_attn_f32_kernel<128>, grid, block, 0, stream, Q, K, V, T, len, O,
                       lse, p, seq, n_tiles);
  else
    hipLaunchKernelGGL(chunk_attn_f32_kernel<64>, grid, block, 0, stream, Q, K, V, T, len, O,
                       lse, p, seq, n_tiles);
  return hipGetLastError();
}

}  // namespace ca
