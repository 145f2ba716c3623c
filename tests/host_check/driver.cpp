// Exercises the C ABI's host code (argument validation, sequence ordering,
// launch parameters, workspace layout) with the kernel launchers replaced by
// stand-ins, under AddressSanitizer and UndefinedBehaviorSanitizer.  Exits 0
// and prints "host check OK" when every expectation holds.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "compact_attn.h"
#include "stubs.hpp"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,     \
              __LINE__, #cond);                                        \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static void* const FAKE = reinterpret_cast<void*>(0x10000);  // never dereferenced by the host code

int main() {
  // ---- union tables: a full batch, then errors
  {
    std::vector<int32_t> nq(CA_MAX_BATCH, 4), nkb(CA_MAX_BATCH, 20);
    nq.back() = 3;
    nkb.back() = 17;
    EXPECT(ca_build_union_tables((const uint8_t*)FAKE, CA_MAX_BATCH, 32, 8, 4, 20, nq.data(),
                                 nkb.data(), (int32_t*)FAKE, (int32_t*)FAKE, 0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "union") == 0);
    EXPECT(stub::last.ints[4] == 3 && stub::last.ints[5] == 17);
    EXPECT(ca_build_union_tables((const uint8_t*)FAKE, CA_MAX_BATCH + 1, 32, 8, 4, 20, nq.data(),
                                 nkb.data(), (int32_t*)FAKE, (int32_t*)FAKE, 0) == CA_ERR_SHAPE);
    nkb[5] = 21;
    EXPECT(ca_build_union_tables((const uint8_t*)FAKE, 8, 32, 8, 4, 20, nq.data(), nkb.data(),
                                 (int32_t*)FAKE, (int32_t*)FAKE, 0) == CA_ERR_SHAPE);
  }
  // ---- attention: ordering longest first, launch parameters, paths
  {
    const int32_t prior[3] = {1024, 8192, 0}, chunk[3] = {256, 128, 64};
    EXPECT(ca_chunk_attention(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE, 200,
                              prior, chunk, 3, 32, 8, 256, 8448, 128, 64, 0.125f, CA_BF16, FAKE,
                              nullptr, 0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "attn_bf16") == 0);
    // dense work (P+C)*C: 327680, 1064960, 4096 -> order 1, 0, 2
    EXPECT(stub::last.seq.order[0] == 1 && stub::last.seq.order[1] == 0 &&
           stub::last.seq.order[2] == 2);
    // 24 (b, g) pairs x 4 workgroups of 8 waves = 96 < 256 CUs: 4-wave workgroups
    EXPECT(stub::last.p.G == 4 && stub::last.p.waves == 4 && stub::last.p.n_t == (4 * 8 + 3) / 4);
    EXPECT(stub::last.p.xcd == 1);  // B*H_kv = 24 is a multiple of 8
    EXPECT(stub::last.p.n_split == 1 && stub::last.p.rows_total == 3LL * 32 * 256);
    EXPECT(ca_chunk_attention(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE, 200,
                              prior, chunk, 3, 32, 8, 256, 8448, 64, 64, 0.125f, CA_F32, FAKE,
                              nullptr, 0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "attn_f32") == 0 && stub::last.D == 64);
    // errors: chunk > C_max, unaligned prior, lse misaligned
    const int32_t bad_chunk[3] = {256, 512, 64};
    EXPECT(ca_chunk_attention(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE, 200,
                              prior, bad_chunk, 3, 32, 8, 256, 8448, 128, 64, 0.125f, CA_BF16, FAKE,
                              nullptr, 0) == CA_ERR_SHAPE);
    const int32_t bad_prior[3] = {1000, 8192, 0};
    EXPECT(ca_chunk_attention(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE, 200,
                              bad_prior, chunk, 3, 32, 8, 256, 8448, 128, 64, 0.125f, CA_BF16,
                              FAKE, nullptr, 0) == CA_ERR_UNSUPPORTED);
    EXPECT(ca_chunk_attention(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE, 200,
                              prior, chunk, 3, 32, 8, 256, 8448, 128, 64, 0.125f, CA_BF16, FAKE,
                              (float*)((char*)FAKE + 2), 0) == CA_ERR_UNSUPPORTED);
    // the 128K shape: 8 (b, g) pairs x 32 workgroups of 8 waves cover the 256 CUs
    const int32_t p1[1] = {129024}, c1[1] = {2048};
    EXPECT(ca_chunk_attention(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE, 2048,
                              p1, c1, 1, 32, 8, 2048, 131072, 128, 64, 0.088f, CA_BF16, FAKE,
                              nullptr, 0) == CA_OK);
    EXPECT(stub::last.p.waves == 8 && stub::last.p.n_t == 32 && stub::last.p.xcd == 1);
    // split: workspace layout and size check
    const size_t need = ca_chunk_attention_workspace_size(3, 32, 256, 128, 4);
    EXPECT(need == 4ull * 3 * 32 * 256 * 130 * 4);
    EXPECT(ca_chunk_attention_split(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE,
                                    200, prior, chunk, 3, 32, 8, 256, 8448, 128, 64, 0.125f,
                                    CA_BF16, 4, FAKE, need, FAKE, nullptr, 0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "attn_bf16_split") == 0 && stub::last.p.n_split == 4);
    EXPECT(stub::last.p.n_t == (4 * 8 + 3) / 4);  // split-KV keeps 4-wave workgroups
    EXPECT((char*)stub::last.ptrs[1] - (char*)stub::last.ptrs[0] ==
           (ptrdiff_t)(4LL * 3 * 32 * 256 * 128 * 4));
    EXPECT(ca_chunk_attention_split(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE,
                                    200, prior, chunk, 3, 32, 8, 256, 8448, 128, 64, 0.125f,
                                    CA_BF16, 4, FAKE, need - 1, FAKE, nullptr, 0) == CA_ERR_SHAPE);
    EXPECT(ca_chunk_attention_split(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE,
                                    200, prior, chunk, 3, 32, 8, 256, 8448, 128, 64, 0.125f,
                                    CA_F32, 4, FAKE, need, FAKE, nullptr, 0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "attn_f32_split") == 0 && stub::last.p.n_split == 4);
    EXPECT((char*)stub::last.ptrs[1] - (char*)stub::last.ptrs[0] ==
           (ptrdiff_t)(4LL * 3 * 32 * 256 * 128 * 4));
    // device lengths: the host reads none of them; sequences in index order, the
    // kernels get the device pointers
    {
      const int32_t* dp = reinterpret_cast<const int32_t*>(static_cast<uintptr_t>(0x7000100));
      const int32_t* dc = reinterpret_cast<const int32_t*>(static_cast<uintptr_t>(0x7000200));
      EXPECT(ca_chunk_attention_devlen(FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                       (const int32_t*)FAKE, 200, dp, dc, 3, 32, 8, 256, 8448,
                                       128, 64, 0.125f, CA_BF16, FAKE, nullptr, 0) == CA_OK);
      EXPECT(strcmp(stub::last.what, "attn_bf16") == 0);
      EXPECT(stub::last.p.dev_prior == dp && stub::last.p.dev_chunk == dc);
      EXPECT(stub::last.seq.order[0] == 0 && stub::last.seq.order[1] == 1 &&
             stub::last.seq.order[2] == 2);
      EXPECT(ca_chunk_attention(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE,
                                200, prior, chunk, 3, 32, 8, 256, 8448, 128, 64, 0.125f, CA_BF16,
                                FAKE, nullptr, 0) == CA_OK);
      EXPECT(stub::last.p.dev_prior == nullptr && stub::last.p.dev_chunk == nullptr);
      EXPECT(ca_build_union_tables_devlen((const uint8_t*)FAKE, 2, 8, 2, 4, 64, dp, dc,
                                          (int32_t*)FAKE, (int32_t*)FAKE, 0) == CA_OK);
      EXPECT(strcmp(stub::last.what, "union") == 0 && stub::last.ptrs[0] == (void*)dp &&
             stub::last.ptrs[1] == (void*)dc);
    }
    // stamped call: the launch gets the record buffer; too small a buffer is
    // refused with the workgroup count reported
    {
      uint32_t* sb = reinterpret_cast<uint32_t*>(static_cast<uintptr_t>(0x7000400));
      const int32_t p1[1] = {129024}, c1[1] = {2048};
      int n_wg = -1;
      EXPECT(ca_chunk_attention_stamped(FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                        (const int32_t*)FAKE, 2048, p1, c1, 1, 32, 8, 2048,
                                        131072, 128, 64, 0.088f, CA_BF16, FAKE, nullptr, sb, 256,
                                        &n_wg, 0) == CA_OK);
      EXPECT(n_wg == 256 && stub::last.p.stamps == sb);
      stub::last = stub::Record{};
      EXPECT(ca_chunk_attention_stamped(FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                        (const int32_t*)FAKE, 2048, p1, c1, 1, 32, 8, 2048,
                                        131072, 128, 64, 0.088f, CA_BF16, FAKE, nullptr, sb, 255,
                                        &n_wg, 0) == CA_ERR_SHAPE);
      EXPECT(n_wg == 256 && strcmp(stub::last.what, "") == 0);
      EXPECT(ca_chunk_attention(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE,
                                2048, p1, c1, 1, 32, 8, 2048, 131072, 128, 64, 0.088f, CA_BF16,
                                FAKE, nullptr, 0) == CA_OK);
      EXPECT(stub::last.p.stamps == nullptr);
    }
    // fused selection: per-batch maxima and the shape reach the launcher
    {
      const int32_t pr[2] = {3072, 1024}, ch[2] = {256, 192};
      EXPECT(ca_select_chunk(FAKE, FAKE, CA_BF16, 2, 8, 2, 256, 4096, 128, pr, ch, 8, 2,
                             (float*)FAKE, 4, (float*)FAKE, 64, (float*)FAKE, (uint8_t*)FAKE,
                             (int32_t*)FAKE, (int32_t*)FAKE, 0) == CA_OK);
      EXPECT(strcmp(stub::last.what, "select") == 0 && stub::last.ints[0] == 4 &&
             stub::last.ints[1] == 48 && stub::last.ints[7] == 8002 && stub::last.ints[6] == 2);
      EXPECT(stub::last.seq.prior[1] == 1024 && stub::last.seq.chunk[1] == 192);
      // the same with the append fused in: the new rows and the V cache reach
      // the launcher, and a missing V cache or a misaligned source is refused
      void* const kn = reinterpret_cast<void*>(static_cast<uintptr_t>(0x7000));
      void* const vc = reinterpret_cast<void*>(static_cast<uintptr_t>(0x9000));
      EXPECT(ca_append_select_chunk(kn, FAKE, FAKE, FAKE, vc, CA_BF16, 2, 8, 2, 256, 4096, 128,
                                    pr, ch, 8, 2, (float*)FAKE, 4, (float*)FAKE, 64,
                                    (float*)FAKE, (uint8_t*)FAKE, (int32_t*)FAKE,
                                    (int32_t*)FAKE, 0) == CA_OK);
      EXPECT(strcmp(stub::last.what, "append_select") == 0 && stub::last.ptrs[0] == kn &&
             stub::last.ptrs[1] == vc && stub::last.ints[0] == 4 && stub::last.ints[1] == 48);
      stub::last = stub::Record{};
      EXPECT(ca_append_select_chunk(kn, FAKE, FAKE, FAKE, nullptr, CA_BF16, 2, 8, 2, 256, 4096,
                                    128, pr, ch, 8, 2, (float*)FAKE, 4, (float*)FAKE, 64,
                                    (float*)FAKE, (uint8_t*)FAKE, (int32_t*)FAKE,
                                    (int32_t*)FAKE, 0) == CA_ERR_NULL);
      EXPECT(ca_append_select_chunk(reinterpret_cast<void*>(static_cast<uintptr_t>(0x7008)),
                                    FAKE, FAKE, FAKE, vc, CA_BF16, 2, 8, 2, 256, 4096, 128, pr,
                                    ch, 8, 2, (float*)FAKE, 4, (float*)FAKE, 64, (float*)FAKE,
                                    (uint8_t*)FAKE, (int32_t*)FAKE, (int32_t*)FAKE,
                                    0) == CA_ERR_UNSUPPORTED);
      EXPECT(strcmp(stub::last.what, "") == 0);
      // device lengths: nothing read on the host, grids from the caps
      // (chunk_cap = min(C_max, 64 NQ_max) = 256, total_cap = min(L, 64 NKB_max) = 4096)
      const int32_t* const dp = reinterpret_cast<const int32_t*>(static_cast<uintptr_t>(0x5000));
      EXPECT(ca_append_select_chunk_devlen(kn, FAKE, FAKE, FAKE, vc, CA_BF16, 2, 8, 2, 256, 4096,
                                           128, dp, dp + 2, 8, 2, (float*)FAKE, 4, (float*)FAKE,
                                           64, (float*)FAKE, (uint8_t*)FAKE, (int32_t*)FAKE,
                                           (int32_t*)FAKE, 0) == CA_OK);
      EXPECT(strcmp(stub::last.what, "append_select_devlen") == 0 && stub::last.ints[0] == 4 &&
             stub::last.ints[1] == 64 && stub::last.ints[8] == 256 &&
             stub::last.ints[9] == 4096 && stub::last.seq.prior[1] == 0);
      EXPECT(ca_select_chunk_devlen(FAKE, FAKE, CA_BF16, 2, 8, 2, 200, 3000, 128, dp, dp + 2, 8,
                                    2, (float*)FAKE, 4, (float*)FAKE, 64, (float*)FAKE,
                                    (uint8_t*)FAKE, (int32_t*)FAKE, (int32_t*)FAKE, 0) == CA_OK);
      EXPECT(strcmp(stub::last.what, "select_devlen") == 0 && stub::last.ints[0] == 3 &&
             stub::last.ints[8] == 200 && stub::last.ints[9] == 3000);
      stub::last = stub::Record{};
      EXPECT(ca_select_chunk_devlen(FAKE, FAKE, CA_BF16, 2, 8, 2, 256, 4096, 128,
                                    reinterpret_cast<const int32_t*>(static_cast<uintptr_t>(0x5002)),
                                    dp, 8, 2, (float*)FAKE, 4, (float*)FAKE, 64, (float*)FAKE,
                                    (uint8_t*)FAKE, (int32_t*)FAKE, (int32_t*)FAKE,
                                    0) == CA_ERR_UNSUPPORTED);
      EXPECT(strcmp(stub::last.what, "") == 0);
    }
    // no-alloc split: the partials go to the static array (its stand-in address),
    // same layout; a split past the array's size is refused before any launch
    {
      char* const sa = reinterpret_cast<char*>(static_cast<uintptr_t>(0x5c7a7c400000ull));
      stub::last = stub::Record{};
      EXPECT(ca_chunk_attention_split_noalloc(FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                              (const int32_t*)FAKE, 200, prior, chunk, 3, 32, 8,
                                              256, 8448, 128, 64, 0.125f, CA_BF16, 4, FAKE,
                                              nullptr, 0) == CA_OK);
      EXPECT(strcmp(stub::last.what, "attn_bf16_split") == 0 && stub::last.p.n_split == 4);
      EXPECT((char*)stub::last.ptrs[0] == sa);
      EXPECT((char*)stub::last.ptrs[1] - sa == (ptrdiff_t)(4LL * 3 * 32 * 256 * 128 * 4));
      EXPECT(ca_chunk_attention_split_noalloc(FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                              (const int32_t*)FAKE, 200, prior, chunk, 3, 32, 8,
                                              256, 8448, 128, 64, 0.125f, CA_F32, 4, FAKE,
                                              nullptr, 0) == CA_OK);
      EXPECT(strcmp(stub::last.what, "attn_f32_split") == 0 && (char*)stub::last.ptrs[0] == sa);
      stub::last = stub::Record{};
      EXPECT(ca_chunk_attention_split_noalloc(FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                              (const int32_t*)FAKE, 200, prior, chunk, 3, 32, 8,
                                              256, 8448, 128, 64, 0.125f, CA_BF16, 8, FAKE,
                                              nullptr, 0) == CA_ERR_TOO_LARGE);
      EXPECT(strcmp(stub::last.what, "") == 0);
    }
    // balanced: workspace layout (partial tiles for 2 tiles + 1024 parts, then
    // the part numbering), size check, 8-wave tiles, one workgroup per slot,
    // fp32 runs unplanned
    const size_t bneed = ca_chunk_attention_balanced_workspace_size(3, 32, 8, 256, 128);
    const long long units = 3LL * 8 * ((4 * 8 + 7) / 8);
    const long long parts = 2 * units + 1024;
    const long long po = parts * 256 * 128 * 4, pml = parts * 256 * 2 * 4;
    const long long pre_off = ((po + pml + 15) / 16) * 16;
    EXPECT(bneed == (size_t)(((pre_off + (units + 1) * 4) + 15) / 16 * 16));
    EXPECT(ca_chunk_attention_balanced_workspace_size(3, 32, 7, 256, 128) == 0);
    EXPECT(ca_chunk_attention_balanced_workspace_size(3, 32, 8, 256, 96) == 0);
    EXPECT(ca_chunk_attention_balanced(FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                       (const int32_t*)FAKE, 200, prior, chunk, 3, 32, 8, 256,
                                       8448, 128, 64, 0.125f, CA_BF16, FAKE, bneed, FAKE, nullptr,
                                       0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "attn_bf16_balanced") == 0 && stub::last.p.waves == 8 &&
           stub::last.p.n_t == (4 * 8 + 7) / 8 && stub::last.p.xcd == 1);
    EXPECT(stub::last.p.bal_units == units && stub::last.p.bal_parts == parts);
    EXPECT(stub::last.ints[0] >= 1 && stub::last.ints[0] <= 1024);
    EXPECT((char*)stub::last.ptrs[1] - (char*)stub::last.ptrs[0] == (ptrdiff_t)po);
    EXPECT((const char*)stub::last.p.bal_pre - (char*)stub::last.ptrs[0] == (ptrdiff_t)pre_off);
    {  // more tiles than slots: the plain kernel, no workspace needed past 16 bytes
      int32_t p17[17], c17[17];
      for (int i = 0; i < 17; ++i) {
        p17[i] = 64 * i;
        c17[i] = 2048;
      }
      EXPECT(ca_chunk_attention_balanced_workspace_size(17, 64, 8, 2048, 64) == 16);
      EXPECT(ca_chunk_attention_balanced(FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                         (const int32_t*)FAKE, 64, p17, c17, 17, 64, 8, 2048,
                                         4096, 64, 64, 0.125f, CA_BF16, FAKE, 16, FAKE, nullptr,
                                         0) == CA_OK);
      EXPECT(strcmp(stub::last.what, "attn_bf16") == 0);
    }
    EXPECT(ca_chunk_attention_balanced(FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                       (const int32_t*)FAKE, 200, prior, chunk, 3, 32, 8, 256,
                                       8448, 128, 64, 0.125f, CA_BF16, FAKE, bneed - 1, FAKE,
                                       nullptr, 0) == CA_ERR_SHAPE);
    EXPECT(ca_chunk_attention_balanced(FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                       (const int32_t*)FAKE, 200, prior, chunk, 3, 32, 8, 256,
                                       8448, 128, 64, 0.125f, CA_BF16, nullptr, bneed, FAKE,
                                       nullptr, 0) == CA_ERR_NULL);
    EXPECT(ca_chunk_attention_balanced(FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                       (const int32_t*)FAKE, 200, prior, chunk, 3, 32, 8, 256,
                                       8448, 128, 64, 0.125f, CA_F32, nullptr, 0, FAKE, nullptr,
                                       0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "attn_f32") == 0);
    // per-(head, Q-block) lists
    EXPECT(ca_chunk_attention_rows(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE,
                                   4, 200, prior, chunk, 3, 32, 8, 256, 8448, 128, 64, 0.125f,
                                   CA_BF16, FAKE, nullptr, 0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "attn_bf16_rows") == 0 && stub::last.p.NQ_max == 4 &&
           stub::last.p.n_t == 4 * 4);
  }
  // ---- a full batch of sequences through attention
  {
    std::vector<int32_t> prior(CA_MAX_BATCH), chunk(CA_MAX_BATCH);
    for (int b = 0; b < CA_MAX_BATCH; ++b) {
      prior[b] = 64 * (b % 7);
      chunk[b] = 64 * (1 + b % 3);
    }
    EXPECT(ca_chunk_attention(FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE, 16,
                              prior.data(), chunk.data(), CA_MAX_BATCH, 8, 8, 192, 1024, 128, 64,
                              0.125f, CA_BF16, FAKE, nullptr, 0) == CA_OK);
    // the order is a permutation with non-increasing work
    std::vector<int> seen(CA_MAX_BATCH, 0);
    long long prev = -1;
    for (int r = 0; r < CA_MAX_BATCH; ++r) {
      const int b = stub::last.seq.order[r];
      EXPECT(b >= 0 && b < CA_MAX_BATCH);
      if (b < 0 || b >= CA_MAX_BATCH) break;
      seen[b]++;
      const long long w = (long long)(prior[b] + chunk[b]) * chunk[b];
      EXPECT(prev < 0 || w <= prev);
      prev = w;
    }
    for (int b = 0; b < CA_MAX_BATCH; ++b) EXPECT(seen[b] == 1);
  }
  // ---- compaction, pooling, mask producer, CSR
  {
    const int32_t prior[2] = {1024, 64}, chunk[2] = {128, 64};
    EXPECT(ca_compact_kv(FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE, 20, prior, chunk,
                         2, 8, 1280, 128, CA_BF16, FAKE, FAKE, (int32_t*)FAKE, 0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "compact") == 0 && stub::last.ints[3] == 2);
    const int32_t lo[2] = {0, 3}, hi[2] = {16, 5};
    EXPECT(ca_pool_blocks(FAKE, CA_F32, 2, 8, 1280, 64, lo, hi, (float*)FAKE, 20, 0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "pool") == 0 && stub::last.ints[3] == 16 &&
           stub::last.ints[5] == 2);
    const int32_t hi_bad[2] = {16, 21};
    EXPECT(ca_pool_blocks(FAKE, CA_F32, 2, 8, 1280, 64, lo, hi_bad, (float*)FAKE, 20, 0) ==
           CA_ERR_SHAPE);
    EXPECT(ca_block_mask_topk((const float*)FAKE, (const float*)FAKE, 2, 32, 8, 2, 20, 128, prior,
                              chunk, 8, 2, (float*)FAKE, (uint8_t*)FAKE, 0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "mask") == 0 && stub::last.ints[4] == 16);
    EXPECT(ca_block_mask_topk((const float*)FAKE, (const float*)FAKE, 2, 32, 8, 2, 20, 128, prior,
                              chunk, -1, 2, (float*)FAKE, (uint8_t*)FAKE, 0) == CA_ERR_SHAPE);
    EXPECT(ca_tables_to_csr((const int32_t*)FAKE, (const int32_t*)FAKE, 2, 8, 16, 1024,
                            (int32_t*)FAKE, (int32_t*)FAKE, 0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "csr") == 0 && stub::last.ints[0] == 16 &&
           stub::last.ints[2] == 16);
    const int32_t nkb2[2] = {12, 16};
    EXPECT(ca_check_tables((const int32_t*)FAKE, (const int32_t*)FAKE, 2, 8, 16, nkb2,
                           (int32_t*)FAKE, 0) == CA_OK);
    EXPECT(strcmp(stub::last.what, "check") == 0 && stub::last.ints[0] == 16 &&
           stub::last.ints[3] == 16);
    const int32_t nkb_bad[2] = {12, 17};
    EXPECT(ca_check_tables((const int32_t*)FAKE, (const int32_t*)FAKE, 2, 8, 16, nkb_bad,
                           (int32_t*)FAKE, 0) == CA_ERR_SHAPE);
  }
  // ---- status strings for every code and one past the end
  for (int s = 0; s <= 6; ++s) EXPECT(ca_status_string((ca_status)s) != nullptr);
  EXPECT(ca_last_hip_error() != nullptr);

  if (failures) {
    fprintf(stderr, "host check: %d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host check OK\n");
  return 0;
}
