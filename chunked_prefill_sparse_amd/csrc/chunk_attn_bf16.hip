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
//   * A wave owns 32 query rows of one query head; a workgroup (8 waves) owns
//     8 such tiles of one (b, g) pseudo-request, ordered position-major then
//     head, so for G = 4 the 4 heads of a group share two 32-row position
//     blocks and one pass over T[b,g].  Each K/V block staged in LDS feeds
//     256 query rows, so the tile copies per MFMA are half what 4-wave
//     workgroups need (measured 2% faster at 128K than 4 waves, two
//     workgroups per CU).  Shapes that would leave CUs without a workgroup
//     use 4-wave workgroups instead.
//   * Workgroup w runs on XCD w % 8.  When B*H_kv is a multiple of 8, all
//     workgroups of a pseudo-request land on one XCD, so that XCD's L2 serves
//     the block stream its workgroups read in near lockstep.  Sequences are
//     taken longest first.
//   * Causality: keys t <= prior + i.  Blocks above the workgroup's last row
//     are skipped; the token mask is applied only on blocks that straddle a
//     wave's first row.
//
// Data movement
//   * Each listed block's K and V (16 KiB each at D = 128) go from HBM/L2
//     straight into LDS with buffer_load_dwordx4 ... lds through a raw buffer
//     resource over the (b, g) cache slice (no VGPR staging).  K tiles are
//     copied two blocks ahead of use and V tiles one block ahead, each into
//     the free one of two LDS buffers; with 4 or 8 waves a step issues them a
//     quarter at a time between its matrix instructions, and waits for them
//     only at its end.
//   * The table's plain entries are compacted into an LDS list at kernel
//     start, so a step finds its next block with an LDS read.
//   * Both tiles are stored row-major with the 16-byte chunks of each row
//     permuted (XOR swizzle by key); the permutation is applied by choosing
//     each lane's source address, since the DMA writes lanes contiguously.
//   * K is read with ds_read_b128 as the A operand of S^T = K Q^T; V is read
//     with ds_read_b64_tr_b16, which transposes 16-bit elements across each
//     group of 16 lanes, as the A operand of O^T = V^T P^T.  The swizzles make
//     both reads bank-conflict free.
//
// Per block, per wave (D = 128): 16 + 16 v_mfma_f32_32x32x16_bf16.
//   S^T[key][q]: each lane ends with 32 scores of ONE query, so the row max
//   needs only one cross-lane exchange (lanes l, l^32, v_permlane32_swap).
//   Online softmax in fp32 with exp2 (scale * log2 e folded into one FMA);
//   the running max moves only when some lane's block max exceeds it by more
//   than 8 (log2 units), otherwise the stale max is kept (exact: numerator
//   and denominator share it, and every exponent stays <= 2^8).  The
//   probabilities are rounded to bf16 once for P.V; the denominator sums
//   them in fp32 before rounding.  The softmax of one block runs on the
//   vector ALUs between the matrix instructions of the next block's scores
//   and the previous block's P.V, in the same wave.  The score accumulator
//   registers serve directly as the B operand of O^T += V^T P^T: the MFMA
//   contraction index is mapped to keys in the order the accumulator holds
//   them, and the V operand is read in that same key order.

#include <utility>

#include "attn_bf16_common.hpp"

namespace ca {
namespace {

// Instruction interleaving for one pipeline body (scheduling hints only): the
// matrix instructions of S(j1) and then of P.V(j-1) each come with LDS reads
// for the ones ahead and three vector instructions of the softmax of block j,
// which a wave issues while its own matrix instruction runs.  The tile copies
// open the body when a workgroup has two waves; with four or eight, a quarter
// of them opens each quarter of the body, as the step issues them.  Groups
// that cannot be filled are skipped by the scheduler.  (Measured on MI355X: a
// vector instruction of one wave issued while another wave's matrix
// instruction runs overlaps far less than one of the same wave, so the
// softmax belongs inside each wave's matrix phase; three per matrix
// instruction measured best of 2, 3 and 4.)
template <int D, int W, int I>
__device__ __forceinline__ void body_pair() {
  constexpr int DS = D / 16;  // S matrix instructions per key tile
  constexpr int N = kDmaPerWave<D, W>;
  // tile copies after matrix instruction pair I, a quarter of the body apart
  constexpr int qc = W == 2 ? 0
                     : (I == DS / 2 - 1 || I == 3 * DS / 2 - 1) ? N - N / 2
                     : (I == DS - 1)                             ? N / 2
                                                                 : 0;
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
  if constexpr (qc > 0) __builtin_amdgcn_sched_group_barrier(0x020, qc, 0);  // tile copies
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
  __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
  __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
}

template <int D, int W, int... I>
__device__ __forceinline__ void body_pairs(std::integer_sequence<int, I...>) {
  (body_pair<D, W, I>(), ...);
}

template <int D, int W>
__device__ __forceinline__ void body_schedule() {
  constexpr int N = kDmaPerWave<D, W>;
  constexpr int q0 = W == 2 ? 2 * N : N / 2;  // copies ahead of the first reads
  if constexpr (q0 > 0) __builtin_amdgcn_sched_group_barrier(0x020, q0, 0);  // tile copies
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);                          // first reads
  body_pairs<D, W>(std::make_integer_sequence<int, D / 8>{});
}

// W = waves per workgroup.  kRows = false: union tables, T[b,g] shared by the
// W waves (8: one workgroup per CU, two waves per SIMD; 4, two workgroups
// per CU, when 8 would leave CUs idle, and with kSplit).  kRows = true: one table per (b, h, Q-block), the
// per-Q-block lists of a block-sparse kernel, so a workgroup is the 2 waves
// (W = 2) of one 64-row Q-block of one head.
// kSplit = 1: the table of a (b, g) is cut into p.n_split contiguous ranges,
// one per workgroup (the straddling blocks go to the last range), and each
// workgroup writes its unnormalised partial output, running max and
// denominator to part_o / part_ml for split_combine_kernel.  More workgroups
// for shapes with few (b, g) pairs.  kSplit = 2: workgroup w runs the piece
// that a balance plan lists at p.plan_items[w] (sequence and group, tile,
// piece k of n), cut the same way; pieces of an uncut tile (n = 1) write O
// and lse themselves.
template <int D, int W, bool kRows, int kSplit>
__global__ __launch_bounds__(W * 64, 8 / W) void chunk_attn_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int32_t* __restrict__ T, const int32_t* __restrict__ len, __bf16* __restrict__ O,
    float* __restrict__ lse, AttnParams p, SeqInfo seq, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int DS = D / 16;
  constexpr int DT = D / 32;
  constexpr int RB = Tile<D>::kRowBytes;
  constexpr int CH = Tile<D>::kChunks;
  constexpr int NDMA = kDmaPerWave<D, W>;
  constexpr bool kSpread = W >= 4;  // tile copies spread over the step body
  constexpr int kThreads = W * 64;
  static_assert(kRows ? W == 2 : (W == 4 || W == 8), "workgroup shape");
  static_assert(!(kRows && kSplit != 0), "split ranges are for union tables");
  // LDS: two K tiles, two V tiles, then the compacted entry list (below) and
  // per-wave counts for building it.  One array: with the list in a separate
  // LDS object the compiler no longer proves that the tile reads stay clear of
  // the in-flight tile copies and waits for those copies before every read.
  constexpr int kListCap = 4096;
  __shared__ __attribute__((aligned(1024))) char lds[4 * Tile<D>::kBytes + 2 * kListCap + 4 * W];
  uint16_t* const plist = reinterpret_cast<uint16_t*>(lds + 4 * Tile<D>::kBytes);
  int* const wcount = reinterpret_cast<int*>(lds + 4 * Tile<D>::kBytes + 2 * kListCap);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // same value, known uniform
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // stamped calls: the counters at the start (uniform; a scalar read each)
  uint64_t t_start = 0, c_start = 0;
  if (kSplit == 0 && !kRows && p.stamps != nullptr) {
    t_start = __builtin_amdgcn_s_memrealtime();
    c_start = __builtin_amdgcn_s_memtime();
  }
  // ---- workgroup -> (sequence, group, tile[, split])
  const int wg = blockIdx.x;
  int b, g, t;
  int split = 0, n_split = 1;  // this workgroup's range k of n of the tile's plain entries
  if (kSplit == 2) {
    if (wg >= p.plan_items[0]) return;  // past the plan's pieces (uniform)
    const int4 it = reinterpret_cast<const int4*>(p.plan_items)[1 + wg];
    b = it.x / p.H_kv;
    g = it.x - b * p.H_kv;
    t = it.y;
    split = it.z;
    n_split = it.w;
  } else {
    const int n_tt = kSplit ? p.n_t * p.n_split : p.n_t;  // workgroups per (b, g)
    int u;
    if (p.xcd) {
      const int x = wg & 7, k = wg >> 3;
      const int jj = k / n_tt;
      u = x + 8 * jj;
      t = k - jj * n_tt;
    } else {
      u = wg / n_tt;
      t = wg - u * n_tt;
    }
    if (kSplit) {
      n_split = p.n_split;
      split = t / p.n_t;
      t -= split * p.n_t;
    }
    const int rank = u / p.H_kv;
    g = u - rank * p.H_kv;
    b = seq.order[rank];
  }
  const bool partials = kSplit != 0 && n_split > 1;  // else O and lse written here
  int P, C;
  seq_lengths(p, seq, b, P, C);
  const int bg = b * p.H_kv + g;

  const int n_pb = (p.C_max + kRowsPerWave - 1) / kRowsPerWave;
  int pb, h, first_pb, last_pb;
  if (kRows) {  // t -> (Q-block, head): position-major, then head
    const int qb = t / p.G;
    h = g * p.G + (t - qb * p.G);
    pb = 2 * qb + wave;
    first_pb = 2 * qb;
    last_pb = 2 * qb + 1;
  } else {
    const int wt = t * W + wave;
    pb = wt / p.G;
    h = g * p.G + (wt - pb * p.G);
    first_pb = (t * W) / p.G;
    last_pb = (t * W + W - 1) / p.G;
  }
  const bool wave_on = pb < n_pb;
  const int row0 = pb * kRowsPerWave;
  const int row = row0 + l32;
  const bool row_in = wave_on && row < p.C_max;
  const bool row_live = row_in && row < C;
  const size_t qo_row = (static_cast<size_t>(b) * p.H_q + h) * p.C_max + row;

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
  const int kb_limit = (P + last_row) / kBlk;  // last block any row may see
  const int nkb = (P + C + kBlk - 1) / kBlk;   // blocks of this sequence
  // table of the workgroup: T[b,g], or T[b,h,Q-block] for per-Q-block lists
  const size_t trow = kRows ? (static_cast<size_t>(b) * p.H_q + h) * p.NQ_max + first_pb / 2
                            : static_cast<size_t>(bg);
  int nT = len[trow];
  nT = nT < 0 ? 0 : (nT > p.NKB_max ? p.NKB_max : nT);
  const int32_t* __restrict__ Trow = T + trow * p.NKB_max;
  const size_t kv_base = static_cast<size_t>(bg) * static_cast<size_t>(p.L) * D;
  const __bf16* Kbg = K + kv_base;
  const __bf16* Vbg = V + kv_base;

  // ---- per-lane DMA source offsets (bytes within a block) realising the swizzles
  uint32_t offk[NDMA], offv[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int pidx = (i * W + wave) * 64 + lane;  // LDS chunk this lane fills
    const int r = pidx / CH, pc = pidx % CH;
    offk[i] = static_cast<uint32_t>(r * RB + ((pc ^ k_swz<D>(r)) << 4));
    offv[i] = static_cast<uint32_t>(r * RB + ((pc ^ v_swz<D>(r)) << 4));
  }
  // ---- per-lane LDS read offsets
  int k_lane_off[DS];  // K rows l32 (+32), chunk 2s + hh
#pragma unroll
  for (int s = 0; s < DS; ++s) k_lane_off[s] = l32 * RB + (((2 * s + hh) ^ k_swz<D>(l32)) << 4);
  int v_lane_off[DT];  // transposing reads: row 4hh + (lane&15)/4, d quad (lane&3) of half (lane>>4)&1
  {
    const int s16 = lane & 15;
    const int key = 4 * hh + (s16 >> 2);
    const int cl = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      v_lane_off[dt] = key * RB + (((4 * dt + cl) ^ v_swz<D>(key)) << 4) + 8 * (s16 & 1);
  }

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

  WaveState<D> ws;
#pragma unroll
  for (int i = 0; i < DT; ++i) ws.acc[i] = f32x16{};
  ws.m_used = -INFINITY;  // max the exponentials are taken against (raw score units)
  ws.l_part = 0.f;        // this lane half's share of the softmax denominator
  const float c = p.scale_log2;
  const float thr = 8.f / c;
  const int qpos = P + row;  // absolute position of this lane's query

  // Software pipeline over the plain entries (j, j1, j2 = this entry and the
  // next two): K tiles run two blocks ahead of use, V tiles one.  Step for
  // block j (its scores computed and its running max settled): copy K(j2)
  // and V(j) into the free buffers; S(j1) and O += V(j-1) P(j-1) on the
  // matrix cores alongside the probabilities P(j) and the row max of S(j1)
  // on the vector ALUs.  That body has no branches (a copy past the end of
  // the table is turned into an out-of-range buffer read that fetches
  // nothing), so the scheduler can interleave it; the tail then settles the
  // running max for block j1 and looks up the entry after j2.  The loop is
  // unrolled by two so buffer offsets and score registers keep fixed roles.
  // Blocks that need the causal mask come after the loop, one at a time.
  constexpr int TB = Tile<D>::kBytes;
  char* const K0 = lds;
  char* const K1 = lds + TB;
  char* const V0 = lds + 2 * TB;
  char* const V1 = lds + 3 * TB;
  const uint32_t slice_bytes = static_cast<uint32_t>(p.L * D * 2);
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)Kbg, (short)0, slice_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)Vbg, (short)0, slice_bytes, 0x00020000);
  const int row0_wg = first_pb * kRowsPerWave;
  // blocks that reach past the workgroup's first row need the causal mask; with
  // T ascending they are the last entries, [e, nT)
  auto needs_mask = [&](int kb) { return kb * kBlk + kBlk - 1 > P + row0_wg; };
  auto valid = [&](int kb) { return kb >= 0 && kb < nkb && kb <= kb_limit; };
  int e = nT;
  while (e > 0) {
    const int kb = Trow[e - 1];
    if (valid(kb) && !needs_mask(kb)) break;
    --e;
  }
  // The plain entries of [0, e) (valid, no mask needed), compacted into LDS
  // in table order when they fit (block indices below 2^16, at most kListCap
  // of them), so that a step reads the entry after next from LDS, in order
  // with its other LDS reads, rather than by a scalar load it must wait for
  // in its tail (measured 0.8% faster at 128K, 5% on one GPU's
  // tensor-parallel share).  Longer tables walk T itself.
  const bool use_list = e <= kListCap && nkb <= 65536;
  int n_plain = 0;
  if (use_list) {
    for (int c0 = 0; c0 < e; c0 += kThreads) {
      const int pos = c0 + tid;
      const int kb = pos < e ? Trow[pos] : -1;
      const bool pl = pos < e && valid(kb) && !needs_mask(kb);
      const uint64_t m = __ballot(pl);
      if (lane == 0) wcount[wave] = __popcll(m);
      __syncthreads();
      int before = n_plain, total = n_plain;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const int cw = wcount[w];
        before += w < wave ? cw : 0;
        total += cw;
      }
      if (pl) plist[before + __popcll(m & ((1ull << lane) - 1ull))] = static_cast<uint16_t>(kb);
      n_plain = total;
      __syncthreads();
    }
  }
  const int n_all = use_list ? n_plain : e;
  // this workgroup's range of [0, n_all); all of it without splitting
  const int e_lo = static_cast<int>((static_cast<int64_t>(n_all) * split) / n_split);
  const int ee =
      static_cast<int>((static_cast<int64_t>(n_all) * (split + 1)) / n_split);
  auto entry = [&](int jj) -> int {
    return use_list ? __builtin_amdgcn_readfirstlane(static_cast<int>(plist[jj])) : Trow[jj];
  };
  auto next_plain = [&](int jj) {
    if (use_list) return jj;
    while (jj < ee) {
      const int kb = Trow[jj];
      if (valid(kb) && !needs_mask(kb)) break;
      ++jj;
    }
    return jj;
  };

  int j = next_plain(e_lo);
  int j1 = next_plain(j + 1);
  int j2 = next_plain(j1 + 1);
  const int kbj = j < ee ? entry(j) : 0;
  int kb0 = kbj;
  int kb1 = j1 < ee ? entry(j1) : 0;
  int kb2 = j2 < ee ? entry(j2) : 0;
  auto boff = [&](int jj, int kb) {  // block byte offset, or past the end when jj is not used
    return jj < ee ? static_cast<uint32_t>(kb) * (kBlk * D * 2) : slice_bytes;
  };
  f32x16 sa0, sa1, sb0, sb1;  // scores of the current / next block (roles alternate)
  bf16x8 pxa[4], pxb[4];      // probabilities waiting for their P.V (roles alternate)
#pragma unroll
  for (int i = 0; i < 4; ++i) pxa[i] = pxb[i] = bf16x8{};
  if (j < ee) {
    dma_tile<D, W>(K0, krsrc, boff(j, kbj), offk, wave_u);
    dma_tile<D, W>(K1, krsrc, boff(j1, kb1), offk, wave_u);
    // V1 is read by the first step with zero probabilities: make it finite
    uint4* vz = reinterpret_cast<uint4*>(V1);
    for (int i = tid; i < TB / 16; i += kThreads) vz[i] = make_uint4(0u, 0u, 0u, 0u);
    wait_vmem();
    __syncthreads();
    scores<D>(K0, qf, k_lane_off, sa0, sa1);
    update_max<D>(row_max(sa0, sa1), ws, c, thr);
    __syncthreads();  // every wave has read K(j) before its buffer is reused
  }

  // One pipeline step for block j (its scores settled against the running max;
  // P(j-1) waiting in registers):
  //   body  copy K(j2) and V(j) into the free buffers; S(j1) and
  //         O += V(j-1) P(j-1) on the matrix cores; P(j) and the row max of
  //         S(j1) on the vector ALUs.  No branches: a copy past the end of the
  //         table becomes an out-of-range buffer read that fetches nothing.
  //   tail  decide whether S(j1) moves the running max; then, after the
  //         copies have landed, if it does (or at the last step) fold in
  //         V(j) P(j) at once, rescale O and the denominator, and leave zero
  //         probabilities pending.
  // Kin/Vin hold K(j1)/V(j-1); Kfree/Vfree receive K(j2)/V(j).
  auto step = [&](const f32x16& cur0, const f32x16& cur1, f32x16& nxt0, f32x16& nxt1,
                  const bf16x8* pprev, bf16x8* pcur, char* Kin, char* Vin, char* Kfree,
                  char* Vfree) {
    // S(j1) is stale when j1 is past the end: then it is unused
    if (kSpread) {
      // a quarter of the tile copies before each quarter of the matrix work,
      // rather than all of them at once: the copies of all waves entering
      // the memory pipeline together held up the start of their matrix work
      // (measured 2% faster at 128K, 12% on one GPU's tensor-parallel share)
      const uint32_t bk = boff(j2, kb2), bv = boff(j, kb0);
      dma_tile<D, W>(Kfree, krsrc, bk, offk, wave_u, 0, NDMA / 2);
      scores<D>(Kin, qf, k_lane_off, nxt0, nxt1, 0, DS / 2);
      dma_tile<D, W>(Kfree, krsrc, bk, offk, wave_u, NDMA / 2, NDMA);
      scores<D>(Kin, qf, k_lane_off, nxt0, nxt1, DS / 2, DS);
      dma_tile<D, W>(Vfree, vrsrc, bv, offv, wave_u, 0, NDMA / 2);
      accumulate_pv<D>(Vin, pprev, v_lane_off, ws, 0, 2);
      dma_tile<D, W>(Vfree, vrsrc, bv, offv, wave_u, NDMA / 2, NDMA);
      accumulate_pv<D>(Vin, pprev, v_lane_off, ws, 2, 4);
    } else {
      dma_tile<D, W>(Kfree, krsrc, boff(j2, kb2), offk, wave_u);
      dma_tile<D, W>(Vfree, vrsrc, boff(j, kb0), offv, wave_u);
      scores<D>(Kin, qf, k_lane_off, nxt0, nxt1);
      accumulate_pv<D>(Vin, pprev, v_lane_off, ws);
    }
    softmax_probs<D>(cur0, cur1, ws, pcur, c);
    const float mx = row_max(nxt0, nxt1);
    body_schedule<D, W>();
    // Keep P(j) and its denominator in the body: without this the compiler
    // sinks the softmax past the barrier below, out of reach of the matrix
    // instructions it is meant to overlap (measured 2% slower at 128K).
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(pcur[i]));
    asm volatile("" : "+v"(ws.l_part));
    const bool last = j1 >= ee;
    const bool moves = !last && __any(mx > ws.m_used + thr);
    const int j3 = next_plain(j2 + 1);
    const int kb3 = j3 < ee ? entry(j3) : 0;
    wait_vmem();
    __syncthreads();
    if (moves || last) {
      accumulate_pv<D>(Vfree, pcur, v_lane_off, ws);
#pragma unroll
      for (int i = 0; i < 4; ++i) pcur[i] = bf16x8{};
      if (moves) update_max<D>(mx, ws, c, thr);
    }
    j = j1;
    kb0 = kb1;
    j1 = j2;
    kb1 = kb2;
    j2 = j3;
    kb2 = kb3;
  };
  while (j < ee) {
    step(sa0, sa1, sb0, sb1, pxb, pxa, K1, V1, K0, V0);
    if (j >= ee) break;
    step(sb0, sb1, sa0, sa1, pxa, pxb, K0, V0, K1, V1);
  }

  // Blocks that straddle the workgroup's rows (usually one): one at a time,
  // with the causal mask.
  for (int jt = e; jt < (split == n_split - 1 ? nT : e); ++jt) {
    const int kb = Trow[jt];
    if (!valid(kb)) continue;
    __syncthreads();  // every wave is done with the buffers
    dma_tile<D, W>(K0, krsrc, static_cast<uint32_t>(kb) * (kBlk * D * 2), offk, wave_u);
    dma_tile<D, W>(V0, vrsrc, static_cast<uint32_t>(kb) * (kBlk * D * 2), offv, wave_u);
    wait_vmem();
    __syncthreads();
    scores<D>(K0, qf, k_lane_off, sa0, sa1);
    mask_scores(sa0, sa1, kb, hh, qpos);
    update_max<D>(row_max(sa0, sa1), ws, c, thr);
    bf16x8 pf[4];
    softmax_probs<D>(sa0, sa1, ws, pf, c);
    accumulate_pv<D>(V0, pf, v_lane_off, ws);
    __syncthreads();
  }

  if (kSplit == 0 && !kRows && p.stamps != nullptr && tid == 0) {
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
    const uint64_t c_end = __builtin_amdgcn_s_memtime();
    constexpr uint32_t kHwId = 4 | (31 << 11);    // HW_REG_HW_ID, bits 0..31
    constexpr uint32_t kXccId = 20 | (31 << 11);  // HW_REG_XCC_ID
    uint32_t* st = p.stamps + static_cast<size_t>(wg) * kStampWords;
    st[0] = static_cast<uint32_t>(t_start);
    st[1] = static_cast<uint32_t>(t_end - t_start);
    st[2] = static_cast<uint32_t>(c_end - c_start);
    st[3] = (__builtin_amdgcn_s_getreg(kXccId) & 0xFu) |
            (((__builtin_amdgcn_s_getreg(kHwId) >> 8) & 0xFFu) << 8);
  }
  // ---- epilogue: O = acc / l, rows >= C written as 0
  const LaneHalves lh = lane_halves(ws.l_part);
  const float l_tot = lh.lo + lh.hi;
  if (!row_in) return;
  if (partials) {  // partial results: acc (unnormalised), running max, denominator
    if (!row_live) return;
    const size_t prow = static_cast<size_t>(split) * p.rows_total + qo_row;
    float* po = part_o + prow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float* a = reinterpret_cast<const float*>(&ws.acc[dt]) + 4 * rr;
        *reinterpret_cast<float4*>(po + 32 * dt + 8 * rr + 4 * hh) =
            make_float4(a[0], a[1], a[2], a[3]);
      }
    }
    if (hh == 0) *reinterpret_cast<float2*>(part_ml + 2 * prow) = make_float2(ws.m_used, l_tot);
    return;
  }
  const float inv = (row_live && l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (!row_live) {  // padding rows: exact zeros whatever the (unused) Q row held
#pragma unroll
    for (int i = 0; i < DT; ++i) ws.acc[i] = f32x16{};
  }
  __bf16* orow = O + qo_row * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float* a = reinterpret_cast<const float*>(&ws.acc[dt]) + 4 * rr;
      const bf16x2 lo = {static_cast<__bf16>(a[0] * inv), static_cast<__bf16>(a[1] * inv)};
      const bf16x2 hi = {static_cast<__bf16>(a[2] * inv), static_cast<__bf16>(a[3] * inv)};
      u32x2 w;
      w.x = __builtin_bit_cast(uint32_t, lo);
      w.y = __builtin_bit_cast(uint32_t, hi);
      *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * rr + 4 * hh) = w;
    }
  }
  if (lse && hh == 0)
    lse[qo_row] = (row_live && l_tot > 0.f) ? ws.m_used * p.scale + __logf(l_tot) : -INFINITY;
}

}  // namespace

hipError_t launch_chunk_attn_bf16(const void* Q, const void* K, const void* V,
                                  const int32_t* T, const int32_t* len, void* O, float* lse,
                                  int B, int D, const AttnParams& p, const SeqInfo& seq,
                                  hipStream_t stream) {
  const dim3 grid(B * p.H_kv * p.n_t);
  const __bf16* q = static_cast<const __bf16*>(Q);
  const __bf16* k = static_cast<const __bf16*>(K);
  const __bf16* v = static_cast<const __bf16*>(V);
  __bf16* o = static_cast<__bf16*>(O);
  float* const no = nullptr;
  if (p.row_tables) {
    if (D == 128)
      hipLaunchKernelGGL((chunk_attn_bf16_kernel<128, 2, true, 0>), grid, dim3(128), 0, stream,
                         q, k, v, T, len, o, lse, p, seq, no, no);
    else
      hipLaunchKernelGGL((chunk_attn_bf16_kernel<64, 2, true, 0>), grid, dim3(128), 0, stream,
                         q, k, v, T, len, o, lse, p, seq, no, no);
  } else {
    if (p.waves == 8) {
      if (D == 128)
        hipLaunchKernelGGL((chunk_attn_bf16_kernel<128, 8, false, 0>), grid, dim3(512), 0,
                           stream, q, k, v, T, len, o, lse, p, seq, no, no);
      else
        hipLaunchKernelGGL((chunk_attn_bf16_kernel<64, 8, false, 0>), grid, dim3(512), 0,
                           stream, q, k, v, T, len, o, lse, p, seq, no, no);
    } else {
      if (D == 128)
        hipLaunchKernelGGL((chunk_attn_bf16_kernel<128, 4, false, 0>), grid, dim3(256), 0,
                           stream, q, k, v, T, len, o, lse, p, seq, no, no);
      else
        hipLaunchKernelGGL((chunk_attn_bf16_kernel<64, 4, false, 0>), grid, dim3(256), 0,
                           stream, q, k, v, T, len, o, lse, p, seq, no, no);
    }
  }
  return hipGetLastError();
}

namespace {

// Merge of the split partials of one output row per wave: with m_s, l_s, a_s
// the running max (raw score units), denominator and unnormalised output of
// split s and M = max_s m_s, w_s = exp2((m_s - M) * scale * log2 e):
//   O = sum_s w_s a_s / sum_s w_s l_s,   lse = M * scale + log(sum_s w_s l_s).
// Rows past the chunk, and rows no split saw a key for, give O = 0, lse = -inf.
template <int D, typename TOut>
__global__ __launch_bounds__(256) void split_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            AttnParams p, SeqInfo seq,
                                                            TOut* __restrict__ O,
                                                            float* __restrict__ lse) {
  constexpr int E = D / 64;  // elements per lane
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= p.rows_total) return;
  const int lane = threadIdx.x & 63;
  const int64_t per_b = static_cast<int64_t>(p.H_q) * p.C_max;
  const int b = static_cast<int>(r / per_b);
  const int i = static_cast<int>(r % p.C_max);
  int P_b, C_b;
  seq_lengths(p, seq, b, P_b, C_b);
  float M = -INFINITY;
  if (i < C_b)
    for (int sp = 0; sp < p.n_split; ++sp)
      M = fmaxf(M, part_ml[2 * (static_cast<size_t>(sp) * p.rows_total + r)]);
  float acc[E], l = 0.f;
#pragma unroll
  for (int k = 0; k < E; ++k) acc[k] = 0.f;
  if (M != -INFINITY) {
    for (int sp = 0; sp < p.n_split; ++sp) {
      const size_t pr = static_cast<size_t>(sp) * p.rows_total + r;
      const float ms = part_ml[2 * pr];
      if (ms == -INFINITY) continue;
      const float wgt = __builtin_amdgcn_exp2f((ms - M) * p.scale_log2);
      l += wgt * part_ml[2 * pr + 1];
      const float* po = part_o + pr * D + E * lane;
#pragma unroll
      for (int k = 0; k < E; ++k) acc[k] += wgt * po[k];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  TOut* orow = O + r * D + E * lane;
#pragma unroll
  for (int k = 0; k < E; ++k) orow[k] = static_cast<TOut>(acc[k] * inv);
  if (lse && lane == 0) lse[r] = l > 0.f ? M * p.scale + __logf(l) : -INFINITY;
}

// Balance plan for planned pieces of W-wave workgroups, in one workgroup.
//   work(u, t): the table entries that tile t of pseudo-request u = b*H_kv + g
//     walks, from len alone: the entries up to the last block any of its rows
//     may see are all but the chunk's blocks above that block (a table that
//     lacks some of those only makes the estimate high), 0 for a tile of
//     padding rows only.
//   When the longest walk is within 1/8 of the total work per compute unit,
//     nothing is cut (those shapes already balance).  Otherwise walks longer
//     than tau = max(3/4 of the work per compute unit, 16) are cut into
//     min(kMaxPieces, ceil(work / tau)) pieces of even length (measured: tau
//     at the full work per compute unit cut about as many tiles and balanced
//     worse).
//   Pieces are listed longest first (by size class), so the dispatcher, which
//     hands workgroups to compute units in order as they free up, runs a
//     greedy longest-first schedule.
// The piece count is below n_units + 4/3 slots (tau >= 3/4 work / slots).
// The order within a size class depends on atomics and changes no result: a
// piece's work and its partial slot follow from (u, t, k) alone.  Each
// tile's work is kept between the passes in LDS (up to kPlanCached tiles), or
// else in pieces[] (each thread rereads what it wrote), which ends with the
// piece counts.
constexpr int kPlanThreads = 256;
constexpr int kPlanCached = 8192;
constexpr int kPlanClasses = 64;

template <int W>
__global__ __launch_bounds__(kPlanThreads) void balance_plan_kernel(
    const int32_t* __restrict__ len, AttnParams p, SeqInfo seq,
    int n_units, int slots, int32_t* __restrict__ plan, int32_t* __restrict__ pieces) {
  __shared__ unsigned long long s_total;
  __shared__ int s_max;
  __shared__ int s_count[kPlanClasses];
  __shared__ int s_cursor[kPlanClasses];
  __shared__ int s_work[kPlanCached];
  int* const wbuf = n_units <= kPlanCached ? s_work : pieces;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_total = 0ull;
    s_max = 0;
  }
  if (tid < kPlanClasses) s_count[tid] = 0;
  __syncthreads();
  const int n_pb = (p.C_max + kRowsPerWave - 1) / kRowsPerWave;
  auto work = [&](int unit) -> int {
    const int u = unit / p.n_t;
    const int t = unit - u * p.n_t;
    const int b = u / p.H_kv;
    const int P = seq.prior[b], C = seq.chunk[b];
    if ((t * W) / p.G * kRowsPerWave >= C) return 0;
    const int last_pb = min((t * W + W - 1) / p.G, n_pb - 1);
    const int kb_limit = (P + min(C, (last_pb + 1) * kRowsPerWave) - 1) / kBlk;
    const int nkb = (P + C + kBlk - 1) / kBlk;
    // the chunk's own blocks are in the table (its causal block triangle is
    // selected), so the entries past the tile's last visible block are the
    // nkb - 1 - kb_limit chunk blocks above it
    const int n = min(max(len[u], 0), p.NKB_max);
    return max(n - (nkb - 1 - kb_limit), 0);
  };
  unsigned long long part = 0ull;
  int wmax = 0;
  for (int unit = tid; unit < n_units; unit += kPlanThreads) {
    const int w = work(unit);
    wbuf[unit] = w;
    part += static_cast<unsigned long long>(w);
    wmax = max(wmax, w);
  }
  for (int o = 32; o > 0; o >>= 1) {  // wave sums first: one LDS atomic per wave
    part += __shfl_xor(part, o);
    wmax = max(wmax, __shfl_xor(wmax, o));
  }
  if ((tid & 63) == 0) {
    atomicAdd(&s_total, part);
    atomicMax(&s_max, wmax);
  }
  __syncthreads();
  const long long total = static_cast<long long>(s_total);
  wmax = s_max;
  const long long per_slot = (total + slots - 1) / slots;
  // walks are at most NKB_max <= kPlanMaxBlocks entries, so the per-piece
  // arithmetic below stays in 32 bits
  const int tau = 8ll * wmax <= 9ll * per_slot
                      ? INT_MAX
                      : static_cast<int>(max((3ll * total + 4ll * slots - 1) / (4ll * slots), 16ll));
  const int class_step = wmax / kPlanClasses + 1;
  auto n_of = [&](int w) { return w > tau ? min(kMaxPieces, (w - 1) / tau + 1) : 1; };
  auto size_class = [&](int w, int n, int k) {
    const int sz = (w * (k + 1)) / n - (w * k) / n;
    return min(kPlanClasses - 1, sz / class_step);
  };
  for (int unit = tid; unit < n_units; unit += kPlanThreads) {
    const int w = wbuf[unit];
    const int n = n_of(w);
    for (int k = 0; k < n; ++k) atomicAdd(&s_count[size_class(w, n, k)], 1);
  }
  __syncthreads();
  if (tid < 64) {  // longest class first: lane l takes class 63 - l; a scan over lanes
    static_assert(kPlanClasses == 64, "one class per lane");
    const int cnt = s_count[kPlanClasses - 1 - tid];
    int inc = cnt;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (tid >= o) inc += y;
    }
    s_cursor[kPlanClasses - 1 - tid] = inc - cnt;
    if (tid == 63) plan[0] = inc;
  }
  __syncthreads();
  int4* items = reinterpret_cast<int4*>(plan) + 1;
  for (int unit = tid; unit < n_units; unit += kPlanThreads) {
    const int w = wbuf[unit];
    const int n = n_of(w);
    const int u = unit / p.n_t;
    for (int k = 0; k < n; ++k) {
      const int pos = atomicAdd(&s_cursor[size_class(w, n, k)], 1);
      items[pos] = make_int4(u, unit - u * p.n_t, k, n);
    }
    pieces[unit] = n;
  }
}

// Merge of the pieces of cut tiles: workgroup (tile (b, g, t), wave tile w)
// holds the 32 rows that wave w of the tile's attention workgroup owns, one
// row per wave at a time; a tile left whole returns at once (its workgroup
// wrote O and lse).  With m_s, l_s, a_s the running max (raw score units),
// denominator and unnormalised output of piece s, M = max_s m_s and
// w_s = exp2((m_s - M) * scale * log2 e):
//   O = sum_s w_s a_s / sum_s w_s l_s,   lse = M * scale + log(sum_s w_s l_s).
// Every piece's loads of a row are issued before any is used.
constexpr int kCombineThreads = 256;

template <int D, int W>
__global__ __launch_bounds__(kCombineThreads) void plan_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, AttnParams p,
    SeqInfo seq, __bf16* __restrict__ O, float* __restrict__ lse) {
  constexpr int E = D / 64;  // elements per lane
  const int unit = blockIdx.x / W;
  const int n = p.plan_pieces[unit];
  if (n <= 1) return;
  const int u = unit / p.n_t;
  const int t = unit - u * p.n_t;
  const int b = u / p.H_kv;
  const int g = u - b * p.H_kv;
  const int wt = t * W + static_cast<int>(blockIdx.x - unit * W);
  const int pb = wt / p.G;
  const int h = g * p.G + (wt - pb * p.G);
  const int C = seq.chunk[b];
  const int lane = threadIdx.x & 63;
  for (int rr = threadIdx.x >> 6; rr < kRowsPerWave; rr += kCombineThreads / 64) {
    const int i = pb * kRowsPerWave + rr;
    if (i >= p.C_max) break;
    const int64_t r = (static_cast<int64_t>(b) * p.H_q + h) * p.C_max + i;
    float ms[kMaxPieces], ls[kMaxPieces], a[kMaxPieces][E];
#pragma unroll
    for (int sp = 0; sp < kMaxPieces; ++sp) {
      ms[sp] = -INFINITY;
      ls[sp] = 0.f;
#pragma unroll
      for (int k = 0; k < E; ++k) a[sp][k] = 0.f;
      if (sp < n && i < C) {
        const size_t pr = static_cast<size_t>(sp) * p.rows_total + r;
        const float2 ml = *reinterpret_cast<const float2*>(part_ml + 2 * pr);
        ms[sp] = ml.x;
        ls[sp] = ml.y;
        const float* po = part_o + pr * D + E * lane;
#pragma unroll
        for (int k = 0; k < E; ++k) a[sp][k] = po[k];
      }
    }
    float M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < kMaxPieces; ++sp) M = fmaxf(M, ms[sp]);
    float acc[E], l = 0.f;
#pragma unroll
    for (int k = 0; k < E; ++k) acc[k] = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int sp = 0; sp < kMaxPieces; ++sp) {
        if (ms[sp] == -INFINITY) continue;
        const float wgt = __builtin_amdgcn_exp2f((ms[sp] - M) * p.scale_log2);
        l += wgt * ls[sp];
#pragma unroll
        for (int k = 0; k < E; ++k) acc[k] += wgt * a[sp][k];
      }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    __bf16* orow = O + r * D + E * lane;
#pragma unroll
    for (int k = 0; k < E; ++k) orow[k] = static_cast<__bf16>(acc[k] * inv);
    if (lse && lane == 0) lse[r] = l > 0.f ? M * p.scale + __logf(l) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_chunk_attn_bf16_split(const void* Q, const void* K, const void* V,
                                        const int32_t* T, const int32_t* len, void* O,
                                        float* lse, int B, int D, const AttnParams& p,
                                        const SeqInfo& seq, float* part_o, float* part_ml,
                                        hipStream_t stream) {
  const dim3 grid(B * p.H_kv * p.n_t * p.n_split);
  const __bf16* q = static_cast<const __bf16*>(Q);
  const __bf16* k = static_cast<const __bf16*>(K);
  const __bf16* v = static_cast<const __bf16*>(V);
  __bf16* o = static_cast<__bf16*>(O);
  if (D == 128)
    hipLaunchKernelGGL((chunk_attn_bf16_kernel<128, 4, false, 1>), grid, dim3(256), 0, stream,
                       q, k, v, T, len, o, lse, p, seq, part_o, part_ml);
  else
    hipLaunchKernelGGL((chunk_attn_bf16_kernel<64, 4, false, 1>), grid, dim3(256), 0, stream,
                       q, k, v, T, len, o, lse, p, seq, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_split_combine(part_o, part_ml, D, false, o, lse, p, seq, stream);
}

hipError_t launch_chunk_attn_bf16_balanced(const void* Q, const void* K, const void* V,
                                           const int32_t* T, const int32_t* len, void* O,
                                           float* lse, int B, int D, const AttnParams& p,
                                           const SeqInfo& seq, float* part_o, float* part_ml,
                                           hipStream_t stream) {
  const int n_units = B * p.H_kv * p.n_t;
  const int slots = min(p.cus, kPlanMaxSlots);
  int32_t* plan = const_cast<int32_t*>(p.plan_items);
  int32_t* pieces = const_cast<int32_t*>(p.plan_pieces);
  hipLaunchKernelGGL(balance_plan_kernel<8>, dim3(1), dim3(kPlanThreads), 0, stream, len, p,
                     seq, n_units, slots, plan, pieces);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(n_units + 2 * slots);  // at least the plan's pieces
  const __bf16* q = static_cast<const __bf16*>(Q);
  const __bf16* k = static_cast<const __bf16*>(K);
  const __bf16* v = static_cast<const __bf16*>(V);
  __bf16* o = static_cast<__bf16*>(O);
  if (D == 128)
    hipLaunchKernelGGL((chunk_attn_bf16_kernel<128, 8, false, 2>), grid, dim3(512), 0, stream, q,
                       k, v, T, len, o, lse, p, seq, part_o, part_ml);
  else
    hipLaunchKernelGGL((chunk_attn_bf16_kernel<64, 8, false, 2>), grid, dim3(512), 0, stream, q,
                       k, v, T, len, o, lse, p, seq, part_o, part_ml);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cgrid(n_units * 8);  // one workgroup per wave tile of every tile
  if (D == 128)
    hipLaunchKernelGGL((plan_combine_kernel<128, 8>), cgrid, dim3(kCombineThreads), 0, stream,
                       part_o, part_ml, p, seq, o, lse);
  else
    hipLaunchKernelGGL((plan_combine_kernel<64, 8>), cgrid, dim3(kCombineThreads), 0, stream,
                       part_o, part_ml, p, seq, o, lse);
  return hipGetLastError();
}

hipError_t launch_split_combine(const float* part_o, const float* part_ml, int D, bool f32_out,
                                void* O, float* lse, const AttnParams& p, const SeqInfo& seq,
                                hipStream_t stream) {
  const dim3 cgrid(static_cast<unsigned>((p.rows_total + 3) / 4));
  if (f32_out) {
    float* o = static_cast<float*>(O);
    if (D == 128)
      hipLaunchKernelGGL((split_combine_kernel<128, float>), cgrid, dim3(256), 0, stream, part_o,
                         part_ml, p, seq, o, lse);
    else
      hipLaunchKernelGGL((split_combine_kernel<64, float>), cgrid, dim3(256), 0, stream, part_o,
                         part_ml, p, seq, o, lse);
  } else {
    __bf16* o = static_cast<__bf16*>(O);
    if (D == 128)
      hipLaunchKernelGGL((split_combine_kernel<128, __bf16>), cgrid, dim3(256), 0, stream, part_o,
                         part_ml, p, seq, o, lse);
    else
      hipLaunchKernelGGL((split_combine_kernel<64, __bf16>), cgrid, dim3(256), 0, stream, part_o,
                         part_ml, p, seq, o, lse);
  }
  return hipGetLastError();
}

}  // namespace ca
