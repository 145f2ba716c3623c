"""GPU parity at the limits the C ABI documents (include/compact_attn.h).

* A full batch: CA_MAX_BATCH ragged sequences, some with an empty chunk, with
  every output compared against the float64 oracle (union tables bit-exact).
* The union's largest table: NKB_max = 2^19 blocks.
* The bf16 cache slice at its limit: L * D * 2 just under 2^32 bytes, with
  selected blocks at the top of the 32-bit buffer-offset range.
* An fp32 cache slice past 4 GiB (64-bit offsets).

For the two large caches the oracle runs on a compacted copy of the selected
blocks (prior blocks packed to end where the chunk starts, the chunk after
them): attention over it has the same admissible keys and the same causal
relation, so it equals attention over the full cache.
"""
import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from chunked_prefill_sparse_amd._lib import CA_MAX_BATCH
from oracle import chunk_attention_ref, union_tables_ref
from tests.gpu_util import (F32_MAX_ABS, check_lse, Dev, compare_bf16, oracle_full, oracle_tables,
                            say, to_np)

pytestmark = pytest.mark.gpu


def _bern(p):
    return lambda rng, b, H, nq, pb: (rng.random((H, nq, pb)) < p).astype(np.uint8)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_max_batch_ragged(dtype):
    B = CA_MAX_BATCH
    rng = np.random.default_rng(B)
    prior = [64 * int(x) for x in rng.integers(0, 9, B)]
    chunk = [64 * int(x) for x in rng.integers(0, 3, B)]  # 0, 64 or 128 tokens
    chunk[0] = 128
    w = gen.make_custom(B, 4, 2, 64, prior, chunk, dtype, 7, _bern(0.3), C_max=128)
    say(f"max batch {B} {dtype}: {sum(c == 0 for c in chunk)} empty chunks")
    d = Dev(w)
    T, lens = d.tables()
    O, lse = d.attention(T, lens, return_lse=True)
    torch.cuda.synchronize()
    Tr, lr = oracle_tables(w)
    np.testing.assert_array_equal(T.cpu().numpy(), Tr)
    np.testing.assert_array_equal(lens.cpu().numpy(), lr)
    Or, lser = oracle_full(w)
    if dtype == "bf16":
        compare_bf16(to_np(O), Or, "O")
    else:
        assert np.abs(to_np(O) - Or).max() <= F32_MAX_ABS
    live = np.isfinite(lser)
    assert np.array_equal(np.isfinite(to_np(lse)), live)
    check_lse(to_np(lse)[live], lser[live])
    for b in range(B):
        assert np.all(to_np(O)[b, :, chunk[b]:] == 0)


def test_union_at_table_limit():
    NKB = 1 << 19  # the largest NKB_max ca_build_union_tables accepts
    rng = np.random.default_rng(19)
    mask = np.zeros((1, 4, 2, NKB), np.uint8)
    cells = rng.integers(0, NKB, size=(4000,))
    mask[0, rng.integers(0, 4, 4000), rng.integers(0, 2, 4000), cells] = 1
    mask[0, 3, 1, NKB - 1] = 1
    m = torch.from_numpy(mask).cuda()
    T, lens = ca.build_union_tables(m, 2, [2], [NKB])
    torch.cuda.synchronize()
    Tr, lr = union_tables_ref(mask, 2, [2], [NKB])
    np.testing.assert_array_equal(lens.cpu().numpy(), lr)
    np.testing.assert_array_equal(T.cpu().numpy(), Tr)
    with pytest.raises(ca.CompactAttnError):
        ca.build_union_tables(torch.zeros((1, 4, 2, NKB + 64), dtype=torch.uint8, device="cuda"),
                              2, [2], [NKB + 64])


def _large_cache_case(dtype, L, seed):
    """One sequence whose chunk (128 tokens) ends the cache; a sparse mask over
    the prior blocks that includes the first one and the last few; returns
    GPU outputs and the oracle on the compacted selected blocks."""
    D, C, H_q, H_kv = 128, 128, 4, 1
    prior = L - C
    nkb = L // 64
    pblk = prior // 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(seed)
    k = torch.randn((1, H_kv, L, D), generator=g, device="cuda", dtype=torch.float32).to(tdt)
    v = torch.randn((1, H_kv, L, D), generator=g, device="cuda", dtype=torch.float32).to(tdt)
    q = torch.randn((1, H_q, C, D), generator=g, device="cuda", dtype=torch.float32).to(tdt)
    rng = np.random.default_rng(seed)
    mask = np.zeros((1, H_q, C // 64, nkb), np.uint8)
    for h in range(H_q):
        for qb in range(C // 64):
            picks = rng.integers(1, pblk, size=12)
            mask[0, h, qb, picks] = 1
            mask[0, h, qb, 0] = 1
            mask[0, h, qb, pblk - 1 - (h + qb) % 3] = 1  # near the top of the offset range
            mask[0, h, qb, pblk:pblk + qb + 1] = 1       # causal block triangle of the chunk
    m = torch.from_numpy(mask).cuda()
    T, lens = ca.build_union_tables(m, H_kv, [C // 64], [nkb])
    O, lse = ca.chunk_attention(q, k, v, T, lens, [prior], [C], return_lse=True)
    torch.cuda.synchronize()
    Tr, lr = union_tables_ref(mask, H_kv, [C // 64], [nkb])
    np.testing.assert_array_equal(T.cpu().numpy(), Tr)
    np.testing.assert_array_equal(lens.cpu().numpy(), lr)
    sel = Tr[0, 0, :lr[0, 0]]
    assert sel[-1] == nkb - 1 and sel[-3] >= pblk - 3
    idx = torch.from_numpy(sel.astype(np.int64)).cuda()
    kc = k[0, 0].view(nkb, 64, D)[idx].reshape(1, 1, -1, D).float().cpu().numpy()
    vc = v[0, 0].view(nkb, 64, D)[idx].reshape(1, 1, -1, D).float().cpu().numpy()
    n_prior = int((sel < pblk).sum())
    Tc = np.arange(len(sel), dtype=np.int32).reshape(1, 1, -1)
    lc = np.array([[len(sel)]], np.int32)
    Or, lser = chunk_attention_ref(q.float().cpu().numpy(), kc, vc, Tc, lc, [64 * n_prior], [C],
                                   1.0 / np.sqrt(D))
    say(f"  {dtype} L={L}: {len(sel)} selected blocks, top block offset "
        f"{int(sel[-1]) * 64 * D * (2 if dtype == 'bf16' else 4)} bytes")
    del k, v
    torch.cuda.empty_cache()
    return O, lse, Or, lser


def test_bf16_cache_slice_at_32bit_offset_limit():
    # largest multiple of 64 tokens with L * D * 2 <= 2^32 - 1 at D = 128
    L = ((2 ** 32 - 1) // 256) // 64 * 64
    say(f"bf16 cache slice of {L * 256} bytes")
    O, lse, Or, lser = _large_cache_case("bf16", L, 32)
    compare_bf16(to_np(O), Or, "O")
    check_lse(to_np(lse), lser)


def test_f32_cache_slice_past_4gib():
    L = 9 * (1 << 20)  # 9 Mi tokens * 128 * 4 bytes = 4.5 GiB per (b, g) slice
    O, lse, Or, lser = _large_cache_case("f32", L, 33)
    assert np.abs(to_np(O) - Or).max() <= F32_MAX_ABS
    check_lse(to_np(lse), lser, fp32=True)
