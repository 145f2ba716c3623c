// Host-only stand-ins for the kernel launchers, so that the C ABI's host code
// (validation, scheduling metadata, dispatch) can run under AddressSanitizer
// and UndefinedBehaviorSanitizer without a GPU.  Each stub records what it
// was asked to launch and returns hipSuccess.
#include "stubs.hpp"

namespace stub {
Record last;
}

namespace ca {

// Stand-in for the static scratch array's address: a recognisable fake
// pointer, never dereferenced (the launcher stand-ins only record it).
void* static_scratch_address(hipError_t* err) {
  *err = hipSuccess;
  return reinterpret_cast<void*>(static_cast<uintptr_t>(0x5c7a7c400000ull));
}

hipError_t launch_union_tables(const uint8_t*, int B, int H_q, int H_kv, int NQ_max, int NKB_max,
                               const UnionExtents& ext, const int32_t* dev_nq,
                               const int32_t* dev_nkb, int32_t*, int32_t*, int cus,
                               hipStream_t) {
  stub::last = stub::Record{};
  stub::last.what = "union";
  stub::last.B = B;
  stub::last.ints[0] = H_q;
  stub::last.ints[1] = H_kv;
  stub::last.ints[2] = NQ_max;
  stub::last.ints[3] = NKB_max;
  stub::last.ints[4] = ext.nq[B - 1];
  stub::last.ints[5] = ext.nkb[B - 1];
  stub::last.ptrs[0] = const_cast<int32_t*>(dev_nq);
  stub::last.ptrs[1] = const_cast<int32_t*>(dev_nkb);
  stub::last.ints[6] = cus;
  return hipSuccess;
}

hipError_t launch_check_tables(const int32_t*, const int32_t*, int n_bg, int H_kv, int NKB_max,
                               const UnionExtents& ext, int32_t*, hipStream_t) {
  stub::last = stub::Record{};
  stub::last.what = "check";
  stub::last.ints[0] = n_bg;
  stub::last.ints[1] = H_kv;
  stub::last.ints[2] = NKB_max;
  stub::last.ints[3] = ext.nkb[n_bg / H_kv - 1];
  return hipSuccess;
}

hipError_t launch_tables_to_csr(const int32_t*, const int32_t*, int n_bg, int NKB_max,
                                int64_t pages, int32_t*, int32_t*, hipStream_t) {
  stub::last = stub::Record{};
  stub::last.what = "csr";
  stub::last.ints[0] = n_bg;
  stub::last.ints[1] = NKB_max;
  stub::last.ints[2] = static_cast<int>(pages);
  return hipSuccess;
}

static void record_attn(const char* what, int B, int D, const AttnParams& p, const SeqInfo& seq) {
  stub::last = stub::Record{};
  stub::last.what = what;
  stub::last.B = B;
  stub::last.D = D;
  stub::last.p = p;
  stub::last.seq = seq;
}

hipError_t launch_chunk_attn_bf16(const void*, const void*, const void*, const int32_t*,
                                  const int32_t*, void*, float*, int B, int D,
                                  const AttnParams& p, const SeqInfo& seq, hipStream_t) {
  record_attn(p.row_tables ? "attn_bf16_rows" : "attn_bf16", B, D, p, seq);
  return hipSuccess;
}

hipError_t launch_chunk_attn_bf16_split(const void*, const void*, const void*, const int32_t*,
                                        const int32_t*, void*, float*, int B, int D,
                                        const AttnParams& p, const SeqInfo& seq, float* part_o,
                                        float* part_ml, hipStream_t) {
  record_attn("attn_bf16_split", B, D, p, seq);
  stub::last.ptrs[0] = part_o;
  stub::last.ptrs[1] = part_ml;
  return hipSuccess;
}

hipError_t launch_chunk_attn_bf16_balanced(const void*, const void*, const void*,
                                           const int32_t*, const int32_t*, void*, float*, int D,
                                           const AttnParams& p, const SeqInfo& seq,
                                           float* part_o, float* part_ml, int slots,
                                           hipStream_t) {
  record_attn("attn_bf16_balanced", 0, D, p, seq);
  stub::last.ptrs[0] = part_o;
  stub::last.ptrs[1] = part_ml;
  stub::last.ints[0] = slots;
  return hipSuccess;
}

hipError_t launch_chunk_attn_f32(const float*, const float*, const float*, const int32_t*,
                                 const int32_t*, float*, float*, int B, int D,
                                 const AttnParams& p, const SeqInfo& seq, hipStream_t) {
  record_attn(p.row_tables ? "attn_f32_rows" : "attn_f32", B, D, p, seq);
  return hipSuccess;
}

hipError_t launch_chunk_attn_f32_split(const float*, const float*, const float*, const int32_t*,
                                       const int32_t*, float*, float*, int B, int D,
                                       const AttnParams& p, const SeqInfo& seq, float* part_o,
                                       float* part_ml, hipStream_t) {
  record_attn("attn_f32_split", B, D, p, seq);
  stub::last.ptrs[0] = part_o;
  stub::last.ptrs[1] = part_ml;
  return hipSuccess;
}

hipError_t launch_append_kv(const void*, const void*, int B, int H_kv, int C_max, int64_t L,
                            int D, int esz, const SeqInfo& seq, void*, void*, hipStream_t) {
  stub::last = stub::Record{};
  stub::last.what = "append";
  stub::last.B = B;
  stub::last.D = D;
  stub::last.ints[0] = H_kv;
  stub::last.ints[1] = C_max;
  stub::last.ints[2] = static_cast<int>(L);
  stub::last.ints[3] = esz;
  stub::last.seq = seq;
  return hipSuccess;
}

hipError_t launch_select_chunk(const void*, const void*, int esz, int B, int H_q, int H_kv,
                               int C_max, int64_t L, int D, const SeqInfo& seq, int max_nq,
                               int max_pblk, int budget, int local, float*, int NQ_max, float*,
                               int NKB_max, float*, uint8_t*, int32_t*, int32_t*,
                               const AppendSrc* app, const SelLens& dl, hipStream_t) {
  stub::last = stub::Record{};
  stub::last.what = dl.prior ? (app ? "append_select_devlen" : "select_devlen")
                             : (app ? "append_select" : "select");
  stub::last.ints[8] = dl.chunk_cap;
  stub::last.ints[9] = static_cast<int>(dl.total_cap);
  if (app) {
    stub::last.ptrs[0] = const_cast<void*>(app->k_new);
    stub::last.ptrs[1] = app->v_cache;
  }
  stub::last.B = B;
  stub::last.D = D;
  stub::last.ints[0] = max_nq;
  stub::last.ints[1] = max_pblk;
  stub::last.ints[2] = budget;
  stub::last.ints[3] = local;
  stub::last.ints[4] = NQ_max;
  stub::last.ints[5] = NKB_max;
  stub::last.ints[6] = esz;
  stub::last.ints[7] = H_q * 1000 + H_kv;
  stub::last.seq = seq;
  (void)C_max;
  (void)L;
  return hipSuccess;
}

hipError_t launch_union_compact(int n_bg, int NKB_max, int n_rep, int32_t*, int32_t*,
                                hipStream_t) {
  stub::last = stub::Record{};
  stub::last.what = "union_compact";
  stub::last.ints[0] = n_bg;
  stub::last.ints[1] = NKB_max;
  stub::last.ints[2] = n_rep;
  return hipSuccess;
}

hipError_t launch_compact_kv(const void*, const void*, const int32_t*, const int32_t*, int NKB_max,
                             int B, int H_kv, int64_t L, int D, int esz, const SeqInfo& seq,
                             void*, void*, int32_t*, hipStream_t) {
  stub::last = stub::Record{};
  stub::last.what = "compact";
  stub::last.B = B;
  stub::last.D = D;
  stub::last.ints[0] = NKB_max;
  stub::last.ints[1] = H_kv;
  stub::last.ints[2] = static_cast<int>(L);
  stub::last.ints[3] = esz;
  stub::last.seq = seq;
  return hipSuccess;
}

hipError_t launch_pool_blocks(const void*, int esz, int B, int H, int64_t R, int D,
                              const BlockRange& rng, int max_span, float*, int NB_out,
                              hipStream_t) {
  stub::last = stub::Record{};
  stub::last.what = "pool";
  stub::last.B = B;
  stub::last.D = D;
  stub::last.ints[0] = esz;
  stub::last.ints[1] = H;
  stub::last.ints[2] = static_cast<int>(R);
  stub::last.ints[3] = max_span;
  stub::last.ints[4] = NB_out;
  stub::last.ints[5] = rng.end[B - 1] - rng.begin[B - 1];
  return hipSuccess;
}

hipError_t launch_block_mask(const float*, const float*, int B, int H_q, int H_kv, int NQ_max,
                             int NKB_max, int D, const SeqInfo& seq, int max_pblk, int budget,
                             int local, float*, uint8_t*, hipStream_t) {
  stub::last = stub::Record{};
  stub::last.what = "mask";
  stub::last.B = B;
  stub::last.D = D;
  stub::last.ints[0] = H_q;
  stub::last.ints[1] = H_kv;
  stub::last.ints[2] = NQ_max;
  stub::last.ints[3] = NKB_max;
  stub::last.ints[4] = max_pblk;
  stub::last.ints[5] = budget;
  stub::last.ints[6] = local;
  stub::last.seq = seq;
  return hipSuccess;
}

}  // namespace ca
