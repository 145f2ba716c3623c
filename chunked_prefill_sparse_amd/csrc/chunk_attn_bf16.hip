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

// Entries of the compacted list in LDS (see attn_job).
constexpr int kListCap = 4096;

// One job of a workgroup: the rows of tile t of pseudo-request (b, g) over its
// share [lo, hi) of the tile's w work units.  The tile's plain entries are
// split in proportion (entries [n_all lo / w, n_all hi / w)), and the blocks
// that straddle its rows go with the share that ends at w.  A whole tile is
// lo = 0, hi = w = 1.  With partials the job writes its unnormalised output,
// running max and denominator to partial row part_base + the row's index in
// O (kSplit = 1) or + its place in the tile, wave * 32 + row (kSplit = 3);
// else it writes O and lse.
// W = waves per workgroup.  kRows = false: union tables, T[b,g] shared by the
// W waves (8: one workgroup per CU, two waves per SIMD; 4, two workgroups
// per CU, when 8 would leave CUs idle, and with kSplit = 1).  kRows = true: one
// table per (b, h, Q-block), the per-Q-block lists of a block-sparse kernel,
// so a workgroup is the 2 waves (W = 2) of one 64-row Q-block of one head, and
// t = Q-block * G + head in group.
template <int D, int W, bool kRows, int kSplit>
__device__ __forceinline__ void attn_job(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int32_t* __restrict__ T, const int32_t* __restrict__ len, __bf16* __restrict__ O,
    float* __restrict__ lse, const AttnParams& p, const SeqInfo& seq,
    float* __restrict__ part_o, float* __restrict__ part_ml, char* lds, int b, int g, int t,
    int lo, int hi, int w, bool partials, int64_t part_base, uint64_t t_start,
    uint64_t c_start) {
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
  // per-wave counts and last positions for building it, all in the kernel's
  // one array: with the
  // list in a separate LDS object the compiler no longer proves that the tile
  // reads stay clear of the in-flight tile copies and waits for those copies
  // before every read.
  uint16_t* const plist = reinterpret_cast<uint16_t*>(lds + 4 * Tile<D>::kBytes);
  int* const wcount = reinterpret_cast<int*>(lds + 4 * Tile<D>::kBytes + 2 * kListCap);
  int* const wlast = wcount + W;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // same value, known uniform
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

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
  // The plain entries (valid, no mask needed), compacted into LDS in table
  // order when they fit (block indices below 2^16, at most kListCap entries
  // in T), so that a step reads the entry after next from LDS, in order with
  // its other LDS reads, rather than by a scalar load it must wait for in its
  // tail (measured 0.8% faster at 128K, 5% on one GPU's tensor-parallel
  // share).  The same pass finds e, one past the last plain entry: the
  // entries after it, [e, nT), are the ones that need the mask.  Longer
  // tables walk T itself, and find e by a scan from the end.
  const bool use_list = nT <= kListCap && nkb <= 65536;
  int n_plain = 0, e = 0;
  if (use_list) {
    for (int c0 = 0; c0 < nT; c0 += kThreads) {
      const int pos = c0 + tid;
      const int kb = pos < nT ? Trow[pos] : -1;
      const bool pl = pos < nT && valid(kb) && !needs_mask(kb);
      const uint64_t m = __ballot(pl);
      if (lane == 0) {
        wcount[wave] = __popcll(m);
        wlast[wave] = m ? c0 + wave * 64 + 63 - __builtin_clzll(m) : -1;
      }
      __syncthreads();
      int before = n_plain, total = n_plain;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const int cw = wcount[w];
        before += w < wave ? cw : 0;
        total += cw;
        e = max(e, wlast[w] + 1);
      }
      if (pl) plist[before + __popcll(m & ((1ull << lane) - 1ull))] = static_cast<uint16_t>(kb);
      n_plain = total;
      __syncthreads();
    }
  } else {
    e = nT;
    while (e > 0) {
      const int kb = Trow[e - 1];
      if (valid(kb) && !needs_mask(kb)) break;
      --e;
    }
  }
  const int n_all = use_list ? n_plain : e;
  // this workgroup's range of [0, n_all); all of it without splitting
  const int e_lo = static_cast<int>((static_cast<int64_t>(n_all) * lo) / w);
  const int ee = hi >= w ? n_all : static_cast<int>((static_cast<int64_t>(n_all) * hi) / w);
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
  for (int jt = e; jt < (hi >= w ? nT : e); ++jt) {
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
    uint32_t* st = p.stamps + static_cast<size_t>(blockIdx.x) * kStampWords;
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
    const size_t prow = static_cast<size_t>(part_base) +
                        (kSplit == 3 ? static_cast<size_t>(wave * kRowsPerWave + l32) : qo_row);
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

// ---- balanced attention (kSplit = 3)

// LDS of a kernel instance: the job's tiles, entry list and per-wave counts,
// then (kSplit = 3) the plan: work per tile, tail and partial prefix sums,
// spare prefix sums per slot, and a few words of reductions and flags.
constexpr int kPlanMisc = 64;
template <int D, int W>
constexpr int job_lds_bytes() {
  return 4 * Tile<D>::kBytes + 2 * kListCap + 8 * W;
}
constexpr int kJobCap = 16;  // jobs of one slot (at most 11, see balanced_slots)
template <int D, int W, int kSplit>
constexpr int kernel_lds_bytes() {
  return job_lds_bytes<D, W>() +
         (kSplit == 3 ? 4 * (6 * (kPlanMaxSlots + 1) + 4 * kJobCap + kPlanMisc) : 0);
}

// threadIdx.x through an opaque move.  The balanced plan takes its thread
// index from here: lane predicates it computes (lane == 0, tid < n, ...) are
// then not merged with the same predicates in the jobs' code, which would
// keep their lane masks alive through the first job's pipeline, whose
// schedule needs every register.
__device__ __forceinline__ int opaque_tid() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(static_cast<int>(threadIdx.x)));
  return t;
}

// Exclusive prefix sums of K arrays a[k][0, n) (LDS) in place, by all W * 64
// threads of the workgroup (tid: this thread's index; each takes a run of
// consecutive entries); the totals go to total[k].  red: K * W ints of LDS.
template <int W, int K>
__device__ void block_exscan(int* const (&a)[K], int n, int* red, int (&total)[K], int tid) {
  constexpr int kThreads = W * 64;
  const int lane = tid & 63, wave = tid >> 6;
  const int per = (n + kThreads - 1) / kThreads;
  const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
  int sum[K], inc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    sum[k] = 0;
    for (int i = i0; i < i1; ++i) sum[k] += a[k][i];
    inc[k] = sum[k];
  }
  for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int y = __shfl_up(inc[k], o);
      if (lane >= o) inc[k] += y;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < K; ++k) red[k * W + wave] = inc[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    int run = inc[k] - sum[k], tot = 0;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const int r = red[k * W + v];
      run += v < wave ? r : 0;
      tot += r;
    }
    total[k] = tot;
    for (int i = i0; i < i1; ++i) {
      const int x = a[k][i];
      a[k][i] = run;
      run += x;
    }
  }
  __syncthreads();
}

// First index in [0, n) whose value exceeds x (a non-decreasing), else n.
__device__ __forceinline__ int upper_bound_lds(const int* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// Tile i of the balanced plan -> (sequence, group, tile): the tile a plain
// launch runs on workgroup i (pseudo-requests in p's sequence order; with
// p.xcd the tiles of one pseudo-request on one XCD, workgroup i running on
// XCD i % 8).
__device__ __forceinline__ void plan_tile(const AttnParams& p, const SeqInfo& seq, int i, int& b,
                                          int& g, int& t) {
  int u;
  if (p.xcd) {
    const int x = i & 7, k = i >> 3;
    const int jj = k / p.n_t;
    u = x + 8 * jj;
    t = k - jj * p.n_t;
  } else {
    u = i / p.n_t;
    t = i - u * p.n_t;
  }
  const int rank = u / p.H_kv;
  g = u - rank * p.H_kv;
  b = seq.order[rank];
}

// Work units of tile t of (b, g) for the plan: the table entries up to the
// last block any of its rows may see, i.e. all of them but the chunk's blocks
// above that block (a table lacking some of those only makes this high); at
// least 1, so that every tile, one of padding rows only included, gets a job.
template <int W>
__device__ __forceinline__ int tile_work(const AttnParams& p, const SeqInfo& seq,
                                         const int32_t* __restrict__ len, int b, int g, int t) {
  int P, C;
  seq_lengths(p, seq, b, P, C);
  if ((t * W) / p.G * kRowsPerWave >= C) return 1;
  const int n_pb = (p.C_max + kRowsPerWave - 1) / kRowsPerWave;
  const int last_pb = min((t * W + W - 1) / p.G, n_pb - 1);
  const int kb_limit = (P + min(C, (last_pb + 1) * kRowsPerWave) - 1) / kBlk;
  const int nkb = (P + C + kBlk - 1) / kBlk;
  const int n = min(max(len[b * p.H_kv + g], 0), p.NKB_max);
  return max(n - (nkb - 1 - kb_limit), 1);
}

// kSplit = 3: workgroup s of the launch is slot s, one per compute unit, with
// at most as many tiles as slots.  Every workgroup derives the same plan from
// the table lengths, in LDS.  c = kBalJobCost, what a job costs on its own
// (set-up, pipeline fill and drain) in work units:
//   w_i    work units of tile i (tile_work); A = ceil(sum / slots), at least
//          kBalMinShare.  When the longest walk is within 2c of A nothing is
//          cut: slot s runs tile s, as a plain launch would.  Otherwise:
//   heads  slot s first runs tile s (the tile a plain launch runs on workgroup
//          s, so on the same XCD): all of it when w_s - A < max(A/8, 2c),
//          else its first A units;
//   tails  the rest of the cut tiles, laid end to end in tile order, fill the
//          slots' spare capacity A - head_s - c (c kept for the piece's own
//          cost; A grows until the tails fit, and after six rounds the c is
//          dropped, where they always fit), laid end to end in slot order:
//          slot s then runs the tails that fall in its spare range, one piece
//          per tile they cover.
// Tails are at least A/8 long, so a slot runs no more than 11 jobs (its head
// and the at most 10 tails that meet a spare range of length <= A).  A tile
// run in one piece writes O and lse; the pieces of a cut tile (its head, then
// its tail pieces in slot order) write partials, numbered from the prefix sum
// of the piece counts over the cut tiles (at most n + n + slots parts: heads,
// plus a piece per tail and per slot boundary), which slot 0 also writes to
// p.bal_pre for plan_merge_kernel.  The first two jobs of a slot are inlined
// as straight-line code: a loop around the job would keep the values its
// set-up needs live through the previous job's pipeline, past the registers
// the pipeline's schedule needs.  For the same reason the plan takes its
// thread index from opaque_tid, and the jobs read what they need from LDS.
template <int D, int W>
__device__ __forceinline__ void balanced_slots(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int32_t* __restrict__ T, const int32_t* __restrict__ len, __bf16* __restrict__ O,
    float* __restrict__ lse, const AttnParams& p, const SeqInfo& seq,
    float* __restrict__ part_o, float* __restrict__ part_ml, char* lds) {
  constexpr int kThreads = W * 64;
  constexpr int kN = kPlanMaxSlots + 1;
  int* const wk = reinterpret_cast<int*>(lds + job_lds_bytes<D, W>());  // [kN]
  int* const tpre = wk + kN;         // [kN] tail prefix sums (tiles; zero past n)
  int* const spre = tpre + kN;       // [kN] spare prefix sums (slots)
  int* const srank = spre + kN;      // [kN] ranks of the slots with spare capacity
  int* const nzpre = srank + kN;     // [kN] ranks of the tiles with a tail
  int* const bpre = nzpre + kN;      // [kN] part prefix sums
  int* const jobs = bpre + kN;       // [kJobCap][4] this slot's jobs: tile, lo, hi, piece
  int* const misc = jobs + 4 * kJobCap;
  int* const red = misc;             // [4 W] scan totals
  int* const n_jobs = misc + 32;
  int* const parts_fit = misc + 33;  // the parts fit the workspace (always; kept as a guard)
  static_assert(W <= 8, "plan words");
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int n = p.bal_units;
  const int S = static_cast<int>(gridDim.x);

  int sum = 0, mx = 0;
  for (int i = tid; i < n; i += kThreads) {
    int b, g, t;
    plan_tile(p, seq, i, b, g, t);
    const int wv = tile_work<W>(p, seq, len, b, g, t);
    wk[i] = wv;
    sum += wv;
    mx = max(mx, wv);
  }
  for (int o = 32; o > 0; o >>= 1) {
    sum += __shfl_xor(sum, o);
    mx = max(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) {
    red[wave] = sum;
    red[8 + wave] = mx;
  }
  __syncthreads();
  int total = 0, wmax = 0;
#pragma unroll
  for (int v = 0; v < W; ++v) {
    total += red[v];
    wmax = max(wmax, red[8 + v]);
  }
  int A = max((total + S - 1) / S, kBalMinShare);
  const int s = blockIdx.x;
  if (wmax <= A + 2 * kBalJobCost) {
    // nothing cut: slot s runs tile s whole, as a plain launch would
    if (s == 0)
      for (int i = tid; i <= n; i += kThreads) p.bal_pre[i] = 0;
    if (s < n) {
      int b, g, t;
      plan_tile(p, seq, s, b, g, t);
      attn_job<D, W, false, 3>(Q, K, V, T, len, O, lse, p, seq, part_o, part_ml, lds, b, g, t, 0,
                               1, 1, false, 0, 0, 0);
    }
    return;
  }
  int reserve = kBalJobCost;
  auto head_of = [&](int wv) { return wv - A < max(A / 8, 2 * kBalJobCost) ? wv : A; };
  for (int round = 0;; ++round) {
    if (round == 6) {
      reserve = 0;
      break;
    }
    int dem = 0, cap = 0, nsp = 0;
    for (int x = tid; x < S; x += kThreads) {
      const int head = x < n ? head_of(wk[x]) : 0;
      dem += x < n ? wk[x] - head : 0;
      const int spare = max(A - head - reserve, 0);
      cap += spare;
      nsp += spare > 0 ? 1 : 0;
    }
    for (int o = 32; o > 0; o >>= 1) {
      dem += __shfl_xor(dem, o);
      cap += __shfl_xor(cap, o);
      nsp += __shfl_xor(nsp, o);
    }
    __syncthreads();  // every thread is done reading red
    if (lane == 0) {
      red[wave] = dem;
      red[8 + wave] = cap;
      red[16 + wave] = nsp;
    }
    __syncthreads();
    dem = cap = nsp = 0;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      dem += red[v];
      cap += red[8 + v];
      nsp += red[16 + v];
    }
    if (cap >= dem) break;
    A += (dem - cap + max(nsp, 1) - 1) / max(nsp, 1);
  }
  for (int x = tid; x < S; x += kThreads) {  // n <= S
    const int head = x < n ? head_of(wk[x]) : 0;
    const int tail = x < n ? wk[x] - head : 0;
    const int spare = max(A - head - reserve, 0);
    tpre[x] = tail;
    spre[x] = spare;
    srank[x] = spare > 0 ? 1 : 0;
    nzpre[x] = tail > 0 ? 1 : 0;
  }
  __syncthreads();  // (also: every thread has read red)
  {
    int* const arrs[4] = {tpre, spre, srank, nzpre};
    int tot[4];
    block_exscan<W, 4>(arrs, S, red, tot, tid);
    if (tid == 0) {
      tpre[S] = tot[0];
      spre[S] = tot[1];
      srank[S] = tot[2];
      nzpre[S] = tot[3];
    }
  }
  __syncthreads();
  const int tails = tpre[S];
  // the slot whose spare range holds tail unit x (always one with spare
  // capacity), and the rank of a slot among those: a tail over the slots of
  // ranks r0 .. r1 is cut into r1 - r0 + 1 pieces
  auto slot_of = [&](int x) { return upper_bound_lds(spre, S + 1, x) - 1; };
  for (int i = tid; i < n; i += kThreads) {
    const int tail = tpre[i + 1] - tpre[i];
    const int pieces =
        tail > 0 ? 1 + srank[slot_of(tpre[i + 1] - 1)] - srank[slot_of(tpre[i])] + 1 : 1;
    bpre[i] = pieces > 1 ? pieces : 0;
  }
  __syncthreads();
  int parts;
  {
    int* const arrs[1] = {bpre};
    int tot[1];
    block_exscan<W, 1>(arrs, n, red, tot, tid);
    parts = tot[0];
  }
  if (s == 0)  // the part numbering, for the merge
    for (int i = tid; i <= n; i += kThreads) p.bal_pre[i] = i < n ? bpre[i] : parts;
  // this slot's jobs: its head, then one piece for each tile whose tail meets
  // the slot's spare range [x0, x1), in tile order (the tiles with a tail
  // between the first and the last met)
  const int x0 = spre[s], x1 = min(spre[s + 1], tails);
  const int has_head = s < n ? 1 : 0;
  int i_first = 0, n_tail_jobs = 0;
  if (x0 < x1) {
    i_first = upper_bound_lds(tpre, n + 1, x0) - 1;
    const int i_last = upper_bound_lds(tpre, n + 1, x1 - 1) - 1;
    n_tail_jobs = nzpre[i_last + 1] - nzpre[i_first];
  }
  if (tid == 0) {
    bpre[n] = parts;
    *parts_fit = parts <= p.bal_parts ? 1 : 0;
    *n_jobs = min(has_head + n_tail_jobs, kJobCap);
    if (has_head) {
      jobs[0] = s;
      jobs[1] = 0;
      jobs[2] = head_of(wk[s]);
      jobs[3] = 0;
    }
  }
  for (int i = i_first + tid; x0 < x1 && i < n; i += kThreads) {
    const int t0 = tpre[i], t1 = tpre[i + 1];
    if (t0 >= x1) break;
    if (t1 <= t0 || t1 <= x0) continue;
    const int j = has_head + nzpre[i] - nzpre[i_first];
    if (j >= kJobCap) break;
    const int head = wk[i] - (t1 - t0);
    jobs[4 * j] = i;
    jobs[4 * j + 1] = head + max(x0, t0) - t0;
    jobs[4 * j + 2] = head + min(x1, t1) - t0;
    jobs[4 * j + 3] = 1 + srank[s] - srank[slot_of(t0)];
  }
  __syncthreads();

  // job j of this slot: units [lo, hi) of tile i, piece k of the tile
  auto job = [&](int j) __attribute__((always_inline)) {
    const int i = __builtin_amdgcn_readfirstlane(jobs[4 * j]);
    const int lo = __builtin_amdgcn_readfirstlane(jobs[4 * j + 1]);
    const int hi = __builtin_amdgcn_readfirstlane(jobs[4 * j + 2]);
    const int k = __builtin_amdgcn_readfirstlane(jobs[4 * j + 3]);
    const int wv = __builtin_amdgcn_readfirstlane(wk[i]);
    const int b0 = __builtin_amdgcn_readfirstlane(bpre[i]);
    // (values the set-up needs come from LDS, none from registers kept since
    // the plan: a register live through the previous job's pipeline spills)
    const bool cut = __builtin_amdgcn_readfirstlane(bpre[i + 1]) > b0 &&
                     __builtin_amdgcn_readfirstlane(*parts_fit) != 0;
    int b, g, t;
    plan_tile(p, seq, i, b, g, t);
    __syncthreads();  // the previous job is done with the tiles and the list
    attn_job<D, W, false, 3>(Q, K, V, T, len, O, lse, p, seq, part_o, part_ml, lds, b, g, t, lo,
                             hi, wv, cut, static_cast<int64_t>(b0 + k) * (W * kRowsPerWave), 0,
                             0);
  };
  const int nj = __builtin_amdgcn_readfirstlane(*n_jobs);
  if (nj > 0) job(0);
  if (nj > 1) job(1);
  for (int j = 2; j < nj; ++j) job(j);
}

// The kernel: one job per workgroup (a whole tile, or with kSplit = 1 one of
// p.n_split ranges of its table), or with kSplit = 3 a slot of the balanced
// plan.
template <int D, int W, bool kRows, int kSplit>
__global__ __launch_bounds__(W * 64, 8 / W) void chunk_attn_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int32_t* __restrict__ T, const int32_t* __restrict__ len, __bf16* __restrict__ O,
    float* __restrict__ lse, AttnParams p, SeqInfo seq, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(1024))) char lds[kernel_lds_bytes<D, W, kSplit>()];
  // stamped calls: the counters at the start (uniform; a scalar read each)
  uint64_t t_start = 0, c_start = 0;
  if (kSplit == 0 && !kRows && p.stamps != nullptr) {
    t_start = __builtin_amdgcn_s_memrealtime();
    c_start = __builtin_amdgcn_s_memtime();
  }
  if constexpr (kSplit == 3) {
    balanced_slots<D, W>(Q, K, V, T, len, O, lse, p, seq, part_o, part_ml, lds);
  } else {
    // ---- workgroup -> (sequence, group, tile[, split])
    const int wg = blockIdx.x;
    int b, g, t;
    int split = 0, n_split = 1;  // this workgroup's range k of n of the tile's plain entries
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
    attn_job<D, W, kRows, kSplit>(Q, K, V, T, len, O, lse, p, seq, part_o, part_ml, lds, b, g, t,
                                  split, split + 1, n_split, kSplit != 0 && n_split > 1,
                                  static_cast<int64_t>(split) * p.rows_total, t_start, c_start);
  }
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

namespace {

// Merge of the parts of the cut tiles of a balanced call: workgroup
// (tile i, wave tile w) takes the 32 rows that wave w of tile i owns, 8
// threads per row, each with D/8 consecutive columns; a tile left whole
// (p.bal_pre[i + 1] == p.bal_pre[i]) returns at once.  With m_s, l_s, a_s the
// running max (raw score units), denominator and unnormalised output of part
// s, M = max_s m_s and w_s = exp2((m_s - M) * scale * log2 e) (taken in one
// pass, the sums rescaled as the running M grows):
//   O = sum_s w_s a_s / sum_s w_s l_s,   lse = M * scale + log(sum_s w_s l_s).
// Rows past the chunk, and rows no part saw a key for, give O = 0 and
// lse = -inf.
constexpr int kMergeThreads = 256;

template <int D, int W>
__global__ __launch_bounds__(kMergeThreads) void plan_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, AttnParams p,
    SeqInfo seq, __bf16* __restrict__ O, float* __restrict__ lse) {
  constexpr int E = D / 8;                   // columns per thread
  constexpr size_t kPart = W * kRowsPerWave;  // rows per part
  const int i = blockIdx.x / W;
  const int w = blockIdx.x - i * W;
  const int base = p.bal_pre[i];
  const int n = p.bal_pre[i + 1] - base;
  if (n <= 0 || p.bal_pre[p.bal_units] > p.bal_parts) return;
  int b, g, t;
  plan_tile(p, seq, i, b, g, t);
  const int r = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * E;
  const int wt = t * W + w;
  const int pb = wt / p.G;
  const int n_pb = (p.C_max + kRowsPerWave - 1) / kRowsPerWave;
  if (pb >= n_pb) return;
  const int h = g * p.G + (wt - pb * p.G);
  const int row = pb * kRowsPerWave + r;
  if (row >= p.C_max) return;
  int P, C;
  seq_lengths(p, seq, b, P, C);
  const size_t qo_row = (static_cast<size_t>(b) * p.H_q + h) * p.C_max + row;
  const size_t prow0 = static_cast<size_t>(base) * kPart + w * kRowsPerWave + r;
  // one pass over the parts, four at a time (their loads in flight together):
  // the running max M and the sums rescale when a group raises M
  float M = -INFINITY, l = 0.f, acc[E];
#pragma unroll
  for (int k = 0; k < E; ++k) acc[k] = 0.f;
  for (int s0 = 0; row < C && s0 < n; s0 += 4) {
    float2 ml[4];
    float4 v[4][E / 4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t pr = prow0 + static_cast<size_t>(s0 + u) * kPart;
      const bool in = s0 + u < n;
      ml[u] = in ? *reinterpret_cast<const float2*>(part_ml + 2 * pr) : make_float2(-INFINITY, 0.f);
      const float4* src = reinterpret_cast<const float4*>(part_o + pr * D + c0);
#pragma unroll
      for (int k = 0; k < E / 4; ++k) v[u][k] = in ? src[k] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mn = M;
#pragma unroll
    for (int u = 0; u < 4; ++u) mn = fmaxf(mn, ml[u].x);
    if (mn == -INFINITY) continue;
    const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((M - mn) * p.scale_log2);
    l *= sc;
#pragma unroll
    for (int k = 0; k < E; ++k) acc[k] *= sc;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wgt = ml[u].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((ml[u].x - mn) * p.scale_log2);
      l += wgt * ml[u].y;
#pragma unroll
      for (int k = 0; k < E / 4; ++k) {
        acc[4 * k] += wgt * v[u][k].x;
        acc[4 * k + 1] += wgt * v[u][k].y;
        acc[4 * k + 2] += wgt * v[u][k].z;
        acc[4 * k + 3] += wgt * v[u][k].w;
      }
    }
    M = mn;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint32_t* dst = reinterpret_cast<uint32_t*>(O + qo_row * D + c0);
#pragma unroll
  for (int k = 0; k < E / 2; ++k) {
    const bf16x2 v2 = {static_cast<__bf16>(acc[2 * k] * inv), static_cast<__bf16>(acc[2 * k + 1] * inv)};
    dst[k] = __builtin_bit_cast(uint32_t, v2);
  }
  if (lse && (threadIdx.x & 7) == 0) lse[qo_row] = l > 0.f ? M * p.scale + __logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_chunk_attn_bf16_balanced(const void* Q, const void* K, const void* V,
                                           const int32_t* T, const int32_t* len, void* O,
                                           float* lse, int D, const AttnParams& p,
                                           const SeqInfo& seq, float* part_o, float* part_ml,
                                           int slots, hipStream_t stream) {
  const dim3 grid(slots);  // one workgroup per compute unit
  const __bf16* q = static_cast<const __bf16*>(Q);
  const __bf16* k = static_cast<const __bf16*>(K);
  const __bf16* v = static_cast<const __bf16*>(V);
  __bf16* o = static_cast<__bf16*>(O);
  if (D == 128)
    hipLaunchKernelGGL((chunk_attn_bf16_kernel<128, 8, false, 3>), grid, dim3(512), 0, stream, q,
                       k, v, T, len, o, lse, p, seq, part_o, part_ml);
  else
    hipLaunchKernelGGL((chunk_attn_bf16_kernel<64, 8, false, 3>), grid, dim3(512), 0, stream, q,
                       k, v, T, len, o, lse, p, seq, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 mgrid(static_cast<unsigned>(p.bal_units) * 8);  // one workgroup per wave tile
  if (D == 128)
    hipLaunchKernelGGL((plan_merge_kernel<128, 8>), mgrid, dim3(kMergeThreads), 0, stream,
                       part_o, part_ml, p, seq, o, lse);
  else
    hipLaunchKernelGGL((plan_merge_kernel<64, 8>), mgrid, dim3(kMergeThreads), 0, stream,
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
