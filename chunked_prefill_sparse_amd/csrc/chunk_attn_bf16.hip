// Zero-copy paged chunk attention, bf16 on the gfx950 matrix cores.
//
// CompactAttention, execution stage ("Methodology" of the technical
// summaries): the per-group block table is metadata for a paged *dense*
// attention kernel that reads the selected KV blocks in place from the
// KV-head-major cache [B, H_kv, L, D], where one (batch, KV head, block)
// triple is one contiguous 64*D*2-byte region.  No KV is gathered or
// compacted: the kernel walks T[b,g] and streams each listed block straight
// from the cache into LDS.
//
// Work decomposition
//   * A wave owns 32 query rows of one query head; a workgroup (4 waves) owns
//     4 such tiles of one (b, g) pseudo-request, ordered position-major then
//     head, so for G = 4 the 4 heads of a group share one 32-row position
//     block and one pass over T[b,g].  Each K/V block staged in LDS feeds
//     128 query rows.
//   * Workgroup w runs on XCD w % 8.  When B*H_kv is a multiple of 8, all
//     workgroups of a pseudo-request land on one XCD, so that XCD's L2 serves
//     the block stream its ~64 workgroups read in near lockstep.  Sequences
//     are taken longest first.
//   * Causality: keys t <= prior + i.  Blocks above the workgroup's last row
//     are skipped; the token mask is applied only on blocks that straddle a
//     wave's first row.
//
// Per block, per wave (D = 128):
//   S^T[key][q] = K Q^T : 16 x v_mfma_f32_32x32x16_bf16 (K from LDS as the A
//                 operand, Q held in VGPRs as the B operand).  The transposed
//                 product leaves each lane with 32 scores of ONE query, so the
//                 row max needs only one cross-lane exchange (lanes l, l^32).
//   online softmax in fp32 with exp2 (scale * log2 e folded into one FMA);
//                 the running max is only moved when some lane's block max
//                 exceeds it by more than 8 (log2 units), otherwise the stale
//                 max is kept (exact: numerator and denominator share it, and
//                 every exponent stays <= 2^8).
//   O^T[d][q]  += V^T P^T : 16 x v_mfma_f32_32x32x16_bf16.  The score
//                 accumulator registers are reused directly as the B operand
//                 after rounding to bf16: the MFMA contraction index is mapped
//                 to keys in the order the accumulator already holds them, and
//                 V is written to LDS transposed with the same key order.
//
// LDS (per stage, double buffered): K tile [64][D] row-major with the 16-byte
// chunks of each row XOR-swizzled, and the transposed V tile [D][64] with the
// same kind of swizzle, so that every ds_read_b128 of an MFMA operand is
// bank-conflict free.

#include "kernels.hpp"

namespace ca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlk = 64;      // keys per KV block
constexpr int kThreads = 256; // 4 waves
constexpr int kRowsPerWave = 32;

template <int D>
struct Tile {
  static constexpr int kKBytes = kBlk * D * 2;     // K tile
  static constexpr int kVBytes = kBlk * D * 2;     // V^T tile
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kKLoads = kKBytes / 16 / kThreads;  // 16-byte loads per thread
  static constexpr int kVKeys = D == 128 ? 4 : 2;          // keys per thread for V^T
  static constexpr int kVGroups = kBlk / kVKeys;           // key groups
};

// Byte offset of 16-byte chunk c of K row r.
template <int D>
__device__ __forceinline__ int k_off(int r, int c) {
  if constexpr (D == 128) return r * 256 + ((c ^ (r & 15)) << 4);
  else return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}
// Byte offset of 16-byte chunk c (8 key slots) of V^T row d (64 keys = 128 bytes).
__device__ __forceinline__ int vt_off(int d, int c) { return d * 128 + ((c ^ ((d >> 1) & 7)) << 4); }

// Key slot of key k inside a V^T row: bits 2 and 3 swapped.  The score
// accumulator holds, in lane half h, register r of key tile kt, the key
// 32kt + 8(r/4) + 4h + r%4; slot order makes each lane's 8 contraction values
// for one MFMA (registers 8u..8u+7) contiguous.
__device__ __forceinline__ int key_slot(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

template <int D>
struct Stage {
  uint4 k[Tile<D>::kKLoads];
  uint4 v[Tile<D>::kVKeys];
};

template <int D>
__device__ __forceinline__ void load_stage(Stage<D>& st, const __bf16* __restrict__ Kbg,
                                           const __bf16* __restrict__ Vbg, int kb, int tid) {
  const uint4* ksrc = reinterpret_cast<const uint4*>(Kbg + static_cast<size_t>(kb) * kBlk * D);
#pragma unroll
  for (int i = 0; i < Tile<D>::kKLoads; ++i) st.k[i] = ksrc[tid + i * kThreads];
  constexpr int KV = Tile<D>::kVKeys;
  const int kg = tid % Tile<D>::kVGroups;
  const int dc = tid / Tile<D>::kVGroups;
  const __bf16* vsrc = Vbg + (static_cast<size_t>(kb) * kBlk + kg * KV) * D + dc * 8;
#pragma unroll
  for (int i = 0; i < KV; ++i) st.v[i] = *reinterpret_cast<const uint4*>(vsrc + i * D);
}

template <int D>
__device__ __forceinline__ void store_stage(const Stage<D>& st, char* __restrict__ lds, int tid) {
  constexpr int CH = D / 8;  // 16-byte chunks per K row
#pragma unroll
  for (int i = 0; i < Tile<D>::kKLoads; ++i) {
    const int ci = tid + i * kThreads;
    *reinterpret_cast<uint4*>(lds + k_off<D>(ci / CH, ci % CH)) = st.k[i];
  }
  char* vt = lds + Tile<D>::kKBytes;
  constexpr int KV = Tile<D>::kVKeys;
  const int kg = tid % Tile<D>::kVGroups;
  const int dc = tid / Tile<D>::kVGroups;
  const int slot = key_slot(kg * KV);      // KV consecutive keys -> KV consecutive slots
  const int byte_in_chunk = (slot & 7) * 2;
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&st.v[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&st.v[1]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = dc * 8 + e;
    char* dst = vt + vt_off(d, slot >> 3) + byte_in_chunk;
    const int wi = e >> 1;
    if constexpr (KV == 4) {
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&st.v[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&st.v[3]);
      u32x2 val;
      if (e & 1) { val.x = pack_hi(w0[wi], w1[wi]); val.y = pack_hi(w2[wi], w3[wi]); }
      else       { val.x = pack_lo(w0[wi], w1[wi]); val.y = pack_lo(w2[wi], w3[wi]); }
      *reinterpret_cast<u32x2*>(dst) = val;
    } else {
      *reinterpret_cast<uint32_t*>(dst) = (e & 1) ? pack_hi(w0[wi], w1[wi]) : pack_lo(w0[wi], w1[wi]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void chunk_attn_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int32_t* __restrict__ T, const int32_t* __restrict__ len, __bf16* __restrict__ O,
    float* __restrict__ lse, AttnParams p, SeqInfo seq) {
  constexpr int DS = D / 16;  // MFMA steps along D for S
  constexpr int DT = D / 32;  // 32-row output tiles of O^T
  __shared__ __attribute__((aligned(16))) char smem[2 * Tile<D>::kStage];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- workgroup -> (sequence, group, tile)
  const int wg = blockIdx.x;
  int u, t;
  if (p.xcd) {
    const int x = wg & 7, k = wg >> 3;
    const int jj = k / p.n_t;
    u = x + 8 * jj;
    t = k - jj * p.n_t;
  } else {
    u = wg / p.n_t;
    t = wg - u * p.n_t;
  }
  const int rank = u / p.H_kv;
  const int g = u - rank * p.H_kv;
  const int b = seq.order[rank];
  const int P = seq.prior[b];
  const int C = seq.chunk[b];
  const int bg = b * p.H_kv + g;

  const int n_pb = (p.C_max + kRowsPerWave - 1) / kRowsPerWave;
  const int wt = t * 4 + wave;
  const int pb = wt / p.G;
  const int h = g * p.G + (wt - pb * p.G);
  const bool wave_on = pb < n_pb;
  const int row0 = pb * kRowsPerWave;
  const int row = row0 + l32;
  const bool row_in = wave_on && row < p.C_max;
  const bool row_live = row_in && row < C;
  const size_t qo_row = (static_cast<size_t>(b) * p.H_q + h) * p.C_max + row;

  // rows of this workgroup that attend: [first_pb*32, min(C, (last_pb+1)*32))
  const int first_pb = (t * 4) / p.G;
  int last_pb = (t * 4 + 3) / p.G;
  last_pb = last_pb < n_pb - 1 ? last_pb : n_pb - 1;
  if (first_pb * kRowsPerWave >= C) {  // padding rows only: O = 0, lse = -inf
    if (row_in) {
      uint2* dst = reinterpret_cast<uint2*>(O + qo_row * D);
#pragma unroll
      for (int i = hh; i < D / 4; i += 2) dst[i] = make_uint2(0u, 0u);
      if (lse && hh == 0) lse[qo_row] = -INFINITY;
    }
    return;
  }
  const int last_row = min(C, (last_pb + 1) * kRowsPerWave) - 1;
  const int kb_limit = (P + last_row) / kBlk;            // last block any row may see
  const int nkb = (P + C + kBlk - 1) / kBlk;             // blocks of this sequence
  int nT = len[bg];
  nT = nT < 0 ? 0 : (nT > p.NKB_max ? p.NKB_max : nT);
  const int32_t* __restrict__ Trow = T + static_cast<size_t>(bg) * p.NKB_max;
  const size_t kv_base = static_cast<size_t>(bg) * static_cast<size_t>(p.L) * D;
  const __bf16* Kbg = K + kv_base;
  const __bf16* Vbg = V + kv_base;

  // ---- Q fragments (B operand of S^T = K Q^T): row l32, d = 16s + 8hh + 0..7
  bf16x8 qf[DS];
  if (row_in) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(Q + qo_row * D + 8 * hh);
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = src[2 * s];
  } else {
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = bf16x8{};
  }

  f32x16 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x16{};
  float m_used = -INFINITY;  // max the exponentials are taken against (raw score units)
  float l_part = 0.f;        // this lane half's share of the softmax denominator
  const float thr = 8.f / p.scale_log2;
  const int qpos = P + row;  // absolute position of this lane's query

  auto next_valid = [&](int j) {
    while (j < nT) {
      const int kb = Trow[j];
      if (kb >= 0 && kb < nkb && kb <= kb_limit) break;
      ++j;
    }
    return j;
  };

  Stage<D> st;
  int j = next_valid(0);
  if (j < nT) {
    load_stage<D>(st, Kbg, Vbg, Trow[j], tid);
    store_stage<D>(st, smem, tid);
  }
  __syncthreads();
  int buf = 0;

  while (j < nT) {
    const int kb = Trow[j];
    const int jn = next_valid(j + 1);
    if (jn < nT) load_stage<D>(st, Kbg, Vbg, Trow[jn], tid);

    const char* Ks = smem + buf * Tile<D>::kStage;
    const char* Vs = Ks + Tile<D>::kKBytes;

    // S^T for keys [0,32) and [32,64) of the block
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(Ks + k_off<D>(l32, 2 * s + hh));
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(Ks + k_off<D>(32 + l32, 2 * s + hh));
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[s], s1, 0, 0, 0);
    }

    // causal mask on blocks that reach past the wave's first row
    if (kb * kBlk + kBlk - 1 > P + row0) {
      const int key0 = kb * kBlk + 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + (r & 3);
        if (key > qpos) s0[r] = -INFINITY;
        if (key + 32 > qpos) s1[r] = -INFINITY;
      }
    }

    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));

    if (__any(mx > m_used + thr)) {
      const float m_new = fmaxf(m_used, mx);
      const float alpha = (m_used == -INFINITY) ? 0.f
                          : __builtin_amdgcn_exp2f((m_used - m_new) * p.scale_log2);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i) acc[i] *= alpha;
      m_used = m_new;
    }
    const float msub = (m_used == -INFINITY) ? 0.f : m_used * p.scale_log2;

    bf16x8 pf[4];  // B operands of O^T += V^T P^T: (kt, u) = (0,0) (0,1) (1,0) (1,1)
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], p.scale_log2, -msub));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], p.scale_log2, -msub));
      lsum += e0 + e1;
      pf[r >> 3][r & 7] = static_cast<__bf16>(e0);
      pf[2 + (r >> 3)][r & 7] = static_cast<__bf16>(e1);
    }
    l_part += lsum;

#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {  // q4 = 2*kt + u -> V^T chunk 4kt + 2u + hh
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vs + vt_off(32 * dt + l32, 2 * q4 + hh));
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[q4], acc[dt], 0, 0, 0);
      }
    }

    if (jn < nT) store_stage<D>(st, smem + (buf ^ 1) * Tile<D>::kStage, tid);
    __syncthreads();
    buf ^= 1;
    j = jn;
  }

  // ---- epilogue: O = acc / l, rows >= C written as 0
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  if (!row_in) return;
  const float inv = (row_live && l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (!row_live) {  // padding rows: exact zeros whatever the (unused) Q row held
#pragma unroll
    for (int i = 0; i < DT; ++i) acc[i] = f32x16{};
  }
  __bf16* orow = O + qo_row * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      u32x2 w;
      const float* a = reinterpret_cast<const float*>(&acc[dt]) + 4 * rr;
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      bf16x2 lo = {static_cast<__bf16>(a[0] * inv), static_cast<__bf16>(a[1] * inv)};
      bf16x2 hi = {static_cast<__bf16>(a[2] * inv), static_cast<__bf16>(a[3] * inv)};
      w.x = __builtin_bit_cast(uint32_t, lo);
      w.y = __builtin_bit_cast(uint32_t, hi);
      *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * rr + 4 * hh) = w;
    }
  }
  if (lse && hh == 0)
    lse[qo_row] = (row_live && l_tot > 0.f) ? m_used * p.scale + __logf(l_tot) : -INFINITY;
}

}  // namespace

hipError_t launch_chunk_attn_bf16(const void* Q, const void* K, const void* V,
                                  const int32_t* T, const int32_t* len, void* O, float* lse,
                                  int B, int D, const AttnParams& p, const SeqInfo& seq,
                                  hipStream_t stream) {
  const dim3 grid(B * p.H_kv * p.n_t), block(kThreads);
  const __bf16* q = static_cast<const __bf16*>(Q);
  const __bf16* k = static_cast<const __bf16*>(K);
  const __bf16* v = static_cast<const __bf16*>(V);
  __bf16* o = static_cast<__bf16*>(O);
  if (D == 128)
    hipLaunchKernelGGL(chunk_attn_bf16_kernel<128>, grid, block, 0, stream, q, k, v, T, len, o,
                       lse, p, seq);
  else
    hipLaunchKernelGGL(chunk_attn_bf16_kernel<64>, grid, block, 0, stream, q, k, v, T, len, o,
                       lse, p, seq);
  return hipGetLastError();
}

}  // namespace ca
