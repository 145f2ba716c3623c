// Device helpers shared by the bf16 chunk-attention kernels (gfx950):
// tile geometry and LDS swizzles, the buffer-resource tile copy into LDS, and
// the per-block building blocks (scores on the matrix cores, causal mask, row
// max, running-max update, probabilities, P.V).  The layout conventions are
// described at the top of chunk_attn_bf16.hip.
#pragma once

#include "kernels.hpp"

namespace ca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int kBlk = 64;       // keys per KV block
constexpr int kRowsPerWave = 32;

template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  static constexpr int kBytes = kBlk * kRowBytes;       // one K or V tile
};

// 1 KiB wave copies per tile per wave, for W waves per workgroup.
template <int D, int W>
constexpr int kDmaPerWave = Tile<D>::kBytes / 1024 / W;

// Chunk permutation of the K tile: chunk c of row r sits at c ^ k_swz(r).
template <int D>
__device__ __forceinline__ int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
// Chunk permutation of the V tile.
template <int D>
__device__ __forceinline__ int v_swz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Issue the copy of one 64-row tile (K or V block kb) into LDS through a raw
// buffer resource over the (b, g) cache slice: per-lane 32-bit offsets, the
// block offset in an SGPR, and hardware bounds checking (a block offset at or
// past the slice end reads zeros and touches no memory).  The LDS destination
// of each wave copy is uniform (M0).  Wave copies i0 .. i1-1 of the tile (all
// by default), so that callers can spread a tile's copies over a step.
template <int D, int W>
__device__ __forceinline__ void dma_tile(char* lds_tile, __amdgpu_buffer_rsrc_t rsrc,
                                         uint32_t block_off, const uint32_t* __restrict__ off,
                                         int wave_u, int i0 = 0, int i1 = kDmaPerWave<D, W>) {
#pragma unroll
  for (int i = i0; i < i1; ++i) {
    char* dst = lds_tile + (i * W + wave_u) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 16, off[i], block_off, 0, 0);
  }
}

template <int D>
struct WaveState {
  f32x16 acc[D / 32];
  float m_used;
  float l_part;
};

// S^T = K Q^T for the 64 keys of one K tile: s0 = keys 0..31, s1 = keys 32..63,
// over the 16-wide d slices s_begin .. s_end-1 (all by default; the scores
// start from zero at s_begin = 0 and accumulate otherwise).
template <int D>
__device__ __forceinline__ void scores(const char* __restrict__ Ks, const bf16x8* qf,
                                       const int* __restrict__ k_lane_off, f32x16& s0,
                                       f32x16& s1, int s_begin = 0, int s_end = D / 16) {
  constexpr int RB = Tile<D>::kRowBytes;
  if (s_begin == 0) {
    s0 = f32x16{};
    s1 = f32x16{};
  }
#pragma unroll
  for (int s = s_begin; s < s_end; ++s) {
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(Ks + k_lane_off[s]);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(Ks + k_lane_off[s] + 32 * RB);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[s], s1, 0, 0, 0);
  }
}

// Causal mask of one block's scores: key t of this lane's query at absolute
// position qpos is admissible iff t <= qpos.
__device__ __forceinline__ void mask_scores(f32x16& s0, f32x16& s1, int kb, int hh, int qpos) {
  const int key0 = kb * kBlk + 4 * hh;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = key0 + 8 * (r >> 2) + (r & 3);
    if (key > qpos) s0[r] = -INFINITY;
    if (key + 32 > qpos) s1[r] = -INFINITY;
  }
}

// The two lane halves of a wave exchanged with v_permlane32_swap (a VALU
// swap, no LDS round trip): for x in every lane, lo holds x of lane l & 31
// and hi x of lane (l & 31) + 32, so any symmetric combination of lo and hi
// is lane l's value combined with lane l ^ 32's.
struct LaneHalves {
  float lo, hi;
};
__device__ __forceinline__ LaneHalves lane_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return {__builtin_bit_cast(float, static_cast<uint32_t>(r[0])),
          __builtin_bit_cast(float, static_cast<uint32_t>(r[1]))};
}

// Row max of one block's scores: two chains of 3-input maxima (v_max3_f32),
// then the other lane half.
__device__ __forceinline__ float row_max(const f32x16& s0, const f32x16& s1) {
  float ma = __builtin_fmaxf(__builtin_fmaxf(s0[0], s0[1]), s0[2]);
  float mb = __builtin_fmaxf(__builtin_fmaxf(s1[0], s1[1]), s1[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) {
    ma = __builtin_fmaxf(__builtin_fmaxf(ma, s0[r]), s0[r + 1]);
    mb = __builtin_fmaxf(__builtin_fmaxf(mb, s1[r]), s1[r + 1]);
  }
  const float mx = __builtin_fmaxf(__builtin_fmaxf(ma, mb), __builtin_fmaxf(s0[15], s1[15]));
  const LaneHalves h = lane_halves(mx);
  return __builtin_fmaxf(h.lo, h.hi);
}

// Running-max update for a block whose row max is mx: the max moves only when
// some lane's block max exceeds it by more than thr; then the output
// accumulator and the denominator are rescaled, before this block's
// probabilities are formed.
template <int D>
__device__ __forceinline__ void update_max(float mx, WaveState<D>& ws, float c, float thr) {
  constexpr int DT = D / 32;
  if (__any(mx > ws.m_used + thr)) {
    const float m_new = __builtin_fmaxf(ws.m_used, mx);
    const float alpha = (ws.m_used == -INFINITY) ? 0.f
                        : __builtin_amdgcn_exp2f((ws.m_used - m_new) * c);
    ws.l_part *= alpha;
#pragma unroll
    for (int i = 0; i < DT; ++i) ws.acc[i] *= alpha;
    ws.m_used = m_new;
  }
}

// Probabilities against the running max, rounded to bf16 as the B operands of
// O^T += V^T P^T (in (kt, u) order (0,0) (0,1) (1,0) (1,1)), and this lane's
// share of the denominator, summed in fp32 before the rounding (plain adds:
// v_dot2c_f32_bf16 on the rounded pairs does not issue alongside the matrix
// instructions, adds do).  Branch-free.
template <int D>
__device__ __forceinline__ void softmax_probs(const f32x16& s0, const f32x16& s1,
                                              WaveState<D>& ws, bf16x8* pf, float c) {
  const float msub = (ws.m_used == -INFINITY) ? 0.f : ws.m_used * c;
  float lsum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c, -msub));
    const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r + 1], c, -msub));
    const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c, -msub));
    const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r + 1], c, -msub));
    lsum += e0 + e1 + e2 + e3;
    pf[r >> 3][r & 7] = static_cast<__bf16>(e0);
    pf[r >> 3][(r & 7) + 1] = static_cast<__bf16>(e1);
    pf[2 + (r >> 3)][r & 7] = static_cast<__bf16>(e2);
    pf[2 + (r >> 3)][(r & 7) + 1] = static_cast<__bf16>(e3);
  }
  ws.l_part += lsum;
}

// O^T += V^T P^T for one V tile, over the 16-key slices q_begin .. q_end-1
// (all four by default); the V operand of (dt, kt, u) is two transposing
// reads (keys +0..3 and +8..11 of the 16-key slice).
template <int D>
__device__ __forceinline__ void accumulate_pv(const char* __restrict__ Vs, const bf16x8* pf,
                                              const int* __restrict__ v_lane_off,
                                              WaveState<D>& ws, int q_begin = 0, int q_end = 4) {
  constexpr int DT = D / 32;
  constexpr int RB = Tile<D>::kRowBytes;
#pragma unroll
  for (int q4 = q_begin; q4 < q_end; ++q4) {  // q4 = 2*kt + u: keys 16*q4 + ...
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const char* p0 = Vs + v_lane_off[dt] + (16 * q4) * RB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0 + 8 * RB));
      const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      ws.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf[q4],
                                                           ws.acc[dt], 0, 0, 0);
    }
  }
}

}  // namespace
}  // namespace ca
