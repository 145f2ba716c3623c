"""ca_select_chunk (the fused selection step of one chunk: pooling, scores,
top-k mask, union tables in four launches) against the separate calls it
fuses, bit for bit: kbar, qbar, scores, mask, T and len.  The separate calls
are pinned against the oracle in test_gpu_producer.py and test_gpu_union.py;
here the tables are also checked against the oracle's union of the fused
call's own mask."""
import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from oracle import union_tables_ref
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _separate(q, k, prior, chunk, budget, local, NQ, NKB, kbar):
    B, H_q, _, D = q.shape
    H_kv = k.shape[1]
    kbar = kbar.clone()
    ca.pool_blocks(k, [p // 64 for p in prior], [(p + c) // 64 for p, c in zip(prior, chunk)],
                   out=kbar)
    qbar = torch.zeros((B, H_q, NQ, D), dtype=torch.float32, device=q.device)
    ca.pool_blocks(q, [0] * B, [c // 64 for c in chunk], out=qbar)
    scores = torch.zeros((B, H_q, NQ, NKB), dtype=torch.float32, device=q.device)
    mask, scores = ca.block_mask_topk(qbar, kbar, prior, chunk, budget, local, scores=scores)
    T, lens = ca.build_union_tables(mask, H_kv, [c // 64 for c in chunk],
                                    [(p + c) // 64 for p, c in zip(prior, chunk)])
    return kbar, qbar, scores, mask, T, lens


@pytest.mark.parametrize("dtype,D,G", [(torch.bfloat16, 128, 4), (torch.bfloat16, 64, 2),
                                       (torch.float32, 64, 4)])
def test_select_chunk_matches_separate_calls(dtype, D, G):
    B, H_kv, C_max, L = 2, 2, 256, 4096
    H_q = H_kv * G
    prior, chunk = [3072, 1024], [256, 192]
    gq = torch.Generator().manual_seed(97)
    k = torch.randn((B, H_kv, L, D), generator=gq).to(dtype).cuda()
    q = torch.randn((B, H_q, C_max, D), generator=gq).to(dtype).cuda()
    NQ, NKB = C_max // 64, L // 64
    # pooled keys of the earlier chunks (the fused call pools only the new blocks)
    kbar0 = torch.zeros((B, H_kv, NKB, D), dtype=torch.float32, device="cuda")
    ca.pool_blocks(k, [0] * B, [p // 64 for p in prior], out=kbar0)
    for budget, local in ((8, 2), (0, 4), (200, 0)):
        say(f"select_chunk {dtype} D={D} G={G} budget={budget} local={local}")
        ref = _separate(q, k, prior, chunk, budget, local, NQ, NKB, kbar0)
        kbar = kbar0.clone()
        qbar = torch.zeros((B, H_q, NQ, D), dtype=torch.float32, device="cuda")
        scores = torch.zeros((B, H_q, NQ, NKB), dtype=torch.float32, device="cuda")
        mask = torch.full((B, H_q, NQ, NKB), 7, dtype=torch.uint8, device="cuda")
        T = torch.full((B, H_kv, NKB), 12345, dtype=torch.int32, device="cuda")
        lens = torch.full((B, H_kv), -3, dtype=torch.int32, device="cuda")
        ca.select_chunk(q, k, prior, chunk, budget, local, qbar, kbar, scores, mask, T, lens)
        torch.cuda.synchronize()
        for name, got, want in zip(("kbar", "qbar", "scores", "mask", "T", "lens"),
                                   (kbar, qbar, scores, mask, T, lens), ref):
            if name == "scores":  # written only where qb < chunk/64 and kb < prior/64
                for b in range(B):
                    nq, pb = chunk[b] // 64, prior[b] // 64
                    assert torch.equal(got[b, :, :nq, :pb], want[b, :, :nq, :pb]), name
            elif name == "qbar":
                for b in range(B):
                    assert torch.equal(got[b, :, :chunk[b] // 64], want[b, :, :chunk[b] // 64])
            else:
                assert torch.equal(got, want), name
        Tr, lr = union_tables_ref(mask.cpu().numpy(), H_kv, [c // 64 for c in chunk],
                                  [(p + c) // 64 for p, c in zip(prior, chunk)])
        np.testing.assert_array_equal(T.cpu().numpy(), Tr)
        np.testing.assert_array_equal(lens.cpu().numpy(), lr)


def test_select_chunk_over_a_prompt():
    # every chunk of prefill_small through the fused step and the separate calls
    s = gen.make_prefill_stream("prefill_small")
    k = s.k.cuda()
    NQ, NKB = s.C // 64, s.L // 64
    kbar_f = torch.zeros((1, s.H_kv, NKB, s.D), dtype=torch.float32, device="cuda")
    kbar_s = kbar_f.clone()
    qbar = torch.zeros((1, s.H_q, NQ, s.D), dtype=torch.float32, device="cuda")
    scores = torch.zeros((1, s.H_q, NQ, NKB), dtype=torch.float32, device="cuda")
    mask = torch.empty((1, s.H_q, NQ, NKB), dtype=torch.uint8, device="cuda")
    T = torch.empty((1, s.H_kv, NKB), dtype=torch.int32, device="cuda")
    lens = torch.empty((1, s.H_kv), dtype=torch.int32, device="cuda")
    for c in range(s.n_chunks):
        P = c * s.C
        q = s.q_chunk(c).cuda()
        ref = _separate(q, k, [P], [s.C], 4, 2, NQ, NKB, kbar_s)
        kbar_s = ref[0]
        ca.select_chunk(q, k, [P], [s.C], 4, 2, qbar, kbar_f, scores, mask, T, lens)
        torch.cuda.synchronize()
        assert torch.equal(kbar_f, kbar_s) and torch.equal(mask, ref[3])
        assert torch.equal(T, ref[4]) and torch.equal(lens, ref[5]), c


def test_select_chunk_long_rows():
    # a 1M-token cache (16384 blocks): the top-k past its LDS limit, and a union
    # bitmap of 512 words in 16 copies at the tail of each T row
    B, H_kv, G, D, L, C = 1, 1, 2, 64, 16384 * 64, 256
    H_q = H_kv * G
    prior, chunk = [L - C], [C]
    gq = torch.Generator().manual_seed(98)
    k = torch.randn((B, H_kv, L, D), generator=gq).to(torch.bfloat16).cuda()
    q = torch.randn((B, H_q, C, D), generator=gq).to(torch.bfloat16).cuda()
    NQ, NKB = C // 64, L // 64
    kbar0 = torch.zeros((B, H_kv, NKB, D), dtype=torch.float32, device="cuda")
    ca.pool_blocks(k, [0], [prior[0] // 64], out=kbar0)
    say("select_chunk long rows: NKB=16384")
    ref = _separate(q, k, prior, chunk, 100, 4, NQ, NKB, kbar0)
    kbar = kbar0.clone()
    qbar = torch.zeros((B, H_q, NQ, D), dtype=torch.float32, device="cuda")
    scores = torch.zeros((B, H_q, NQ, NKB), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, H_q, NQ, NKB), dtype=torch.uint8, device="cuda")
    T = torch.full((B, H_kv, NKB), 12345, dtype=torch.int32, device="cuda")
    lens = torch.empty((B, H_kv), dtype=torch.int32, device="cuda")
    ca.select_chunk(q, k, prior, chunk, 100, 4, qbar, kbar, scores, mask, T, lens)
    torch.cuda.synchronize()
    for name, got, want in (("kbar", kbar, ref[0]), ("mask", mask, ref[3]), ("T", T, ref[4]),
                            ("lens", lens, ref[5])):
        assert torch.equal(got, want), name
    Tr, lr = union_tables_ref(mask.cpu().numpy(), H_kv, [C // 64], [L // 64])
    np.testing.assert_array_equal(T.cpu().numpy(), Tr)
    np.testing.assert_array_equal(lens.cpu().numpy(), lr)


@pytest.mark.parametrize("L,prior,chunk", [
    (64, [0, 0], [64, 0]),          # one block: one bitmap word, one copy of it
    (128, [64, 0], [64, 128]),      # two blocks: two copies of the one word
    (320, [128, 256], [192, 64]),   # five blocks: five copies
    (2112, [1920, 0], [192, 0]),    # 33 blocks: two words, 16 copies; one sequence empty
])
def test_select_chunk_small_tables(L, prior, chunk):
    # T rows shorter than 16 bitmap copies: the copies take the whole row
    B, H_kv, G, D, C_max = 2, 2, 3, 64, 192
    H_q = H_kv * G
    gq = torch.Generator().manual_seed(99 + L)
    k = torch.randn((B, H_kv, L, D), generator=gq).to(torch.bfloat16).cuda()
    q = torch.randn((B, H_q, C_max, D), generator=gq).to(torch.bfloat16).cuda()
    NQ, NKB = C_max // 64, L // 64
    kbar0 = torch.zeros((B, H_kv, NKB, D), dtype=torch.float32, device="cuda")
    ca.pool_blocks(k, [0] * B, [p // 64 for p in prior], out=kbar0)
    for budget, local in ((1, 0), (2, 1)):
        say(f"select_chunk small tables L={L} prior={prior} chunk={chunk} budget={budget}")
        ref = _separate(q, k, prior, chunk, budget, local, NQ, NKB, kbar0)
        kbar = kbar0.clone()
        qbar = torch.zeros((B, H_q, NQ, D), dtype=torch.float32, device="cuda")
        scores = torch.zeros((B, H_q, NQ, NKB), dtype=torch.float32, device="cuda")
        mask = torch.full((B, H_q, NQ, NKB), 7, dtype=torch.uint8, device="cuda")
        T = torch.full((B, H_kv, NKB), 12345, dtype=torch.int32, device="cuda")
        lens = torch.full((B, H_kv), -3, dtype=torch.int32, device="cuda")
        ca.select_chunk(q, k, prior, chunk, budget, local, qbar, kbar, scores, mask, T, lens)
        torch.cuda.synchronize()
        for name, got, want in (("kbar", kbar, ref[0]), ("mask", mask, ref[3]),
                                ("T", T, ref[4]), ("lens", lens, ref[5])):
            assert torch.equal(got, want), name
        Tr, lr = union_tables_ref(mask.cpu().numpy(), H_kv, [c // 64 for c in chunk],
                                  [(p + c) // 64 for p, c in zip(prior, chunk)])
        np.testing.assert_array_equal(T.cpu().numpy(), Tr)
        np.testing.assert_array_equal(lens.cpu().numpy(), lr)


@pytest.mark.parametrize("dtype,D,G", [(torch.bfloat16, 128, 4), (torch.bfloat16, 64, 2),
                                       (torch.float32, 128, 2), (torch.float32, 64, 4)])
def test_append_select_matches_append_then_select(dtype, D, G):
    # ca_append_select_chunk against ca_append_kv then ca_select_chunk: caches
    # (rows past the chunk untouched), kbar, qbar, scores, mask, T and lens bit
    # for bit; ragged priors and chunks, caches poisoned with NaN beyond the
    # earlier chunks' rows
    B, H_kv, C_max, L = 2, 2, 256, 4096
    H_q = H_kv * G
    prior, chunk = [3072, 1024], [256, 192]
    gq = torch.Generator().manual_seed(131)
    k0 = torch.randn((B, H_kv, L, D), generator=gq).to(dtype)
    v0 = torch.randn((B, H_kv, L, D), generator=gq).to(dtype)
    for b in range(B):
        k0[b, :, prior[b]:] = float("nan")
        v0[b, :, prior[b]:] = float("nan")
    k_new = torch.randn((B, H_kv, C_max, D), generator=gq).to(dtype).cuda()
    v_new = torch.randn((B, H_kv, C_max, D), generator=gq).to(dtype).cuda()
    q = torch.randn((B, H_q, C_max, D), generator=gq).to(dtype).cuda()
    NQ, NKB = C_max // 64, L // 64
    kbar0 = torch.zeros((B, H_kv, NKB, D), dtype=torch.float32, device="cuda")
    ca.pool_blocks(k0.cuda(), [0] * B, [p // 64 for p in prior], out=kbar0)

    def buffers():
        return (k0.cuda(), v0.cuda(), kbar0.clone(),
                torch.zeros((B, H_q, NQ, D), dtype=torch.float32, device="cuda"),
                torch.zeros((B, H_q, NQ, NKB), dtype=torch.float32, device="cuda"),
                torch.full((B, H_q, NQ, NKB), 7, dtype=torch.uint8, device="cuda"),
                torch.full((B, H_kv, NKB), 12345, dtype=torch.int32, device="cuda"),
                torch.full((B, H_kv), -3, dtype=torch.int32, device="cuda"))

    for budget, local in ((8, 2), (0, 4)):
        say(f"append_select_chunk {dtype} D={D} G={G} budget={budget} local={local}")
        kc, vc, kbar, qbar, scores, mask, T, lens = ref = buffers()
        ca.append_kv(k_new, v_new, kc, vc, prior, chunk)
        ca.select_chunk(q, kc, prior, chunk, budget, local, qbar, kbar, scores, mask, T, lens)
        got = buffers()
        kc2, vc2, kbar2, qbar2, scores2, mask2, T2, lens2 = got
        ca.append_select_chunk(k_new, v_new, q, kc2, vc2, prior, chunk, budget, local, qbar2,
                               kbar2, scores2, mask2, T2, lens2)
        torch.cuda.synchronize()
        names = ("k_cache", "v_cache", "kbar", "qbar", "scores", "mask", "T", "lens")
        for name, g, r in zip(names, got, ref):
            if name == "scores":  # written only where qb < chunk/64 and kb < prior/64
                for b in range(B):
                    nq, pb = chunk[b] // 64, prior[b] // 64
                    assert torch.equal(g[b, :, :nq, :pb], r[b, :, :nq, :pb]), name
            elif name in ("k_cache", "v_cache"):  # NaN rows past the chunk stay NaN
                assert torch.equal(torch.nan_to_num(g, nan=1e30), torch.nan_to_num(r, nan=1e30))
                for b in range(B):
                    e = prior[b] + chunk[b]
                    assert bool(torch.isnan(g[b, :, e:].float()).all()), name
                    src = (k_new if name == "k_cache" else v_new)[b, :, :chunk[b]]
                    assert torch.equal(g[b, :, prior[b]:e], src), name
            else:
                assert torch.equal(g, r), name


def test_append_select_rejects_bad_arguments():
    B, H_kv, H_q, C_max, L, D = 1, 2, 4, 128, 1024, 64
    t = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt, device="cuda")
    k_new, v_new, q = t(B, H_kv, C_max, D), t(B, H_kv, C_max, D), t(B, H_q, C_max, D)
    kc, vc = t(B, H_kv, L, D), t(B, H_kv, L, D)
    qbar, kbar = t(B, H_q, 2, D, dt=torch.float32), t(B, H_kv, 16, D, dt=torch.float32)
    scores, mask = t(B, H_q, 2, 16, dt=torch.float32), t(B, H_q, 2, 16, dt=torch.uint8)
    T, lens = t(B, H_kv, 16, dt=torch.int32), t(B, H_kv, dt=torch.int32)
    args = (qbar, kbar, scores, mask, T, lens)
    with pytest.raises(ValueError):  # new rows of another dtype
        ca.append_select_chunk(k_new.float(), v_new, q, kc, vc, [0], [128], 4, 1, *args)
    with pytest.raises(ValueError):  # new rows of the wrong shape
        ca.append_select_chunk(k_new[:, :, :64], v_new, q, kc, vc, [0], [128], 4, 1, *args)
    with pytest.raises(ca.CompactAttnError) as e:  # chunk not a multiple of 64
        ca.append_select_chunk(k_new, v_new, q, kc, vc, [0], [96], 4, 1, *args)
    assert e.value.status == 4
    with pytest.raises(ca.CompactAttnError) as e:  # past the cache
        ca.append_select_chunk(k_new, v_new, q, kc, vc, [960], [128], 4, 1, *args)
    assert e.value.status == 2
