"""GPU parity of the device-length calls (ca_build_union_tables_devlen,
ca_chunk_attention_devlen, ca_select_chunk_devlen, ca_append_select_chunk_devlen),
through the C ABI.

* With valid lengths they equal the host-length calls bit for bit (same
  kernels) and the oracle within the parity bounds.
* Lengths that break a call's limits make that sequence empty (table len 0;
  O = 0, lse = -inf) and leave the other sequences unchanged.
* One HIP graph holding both calls, captured once, replayed for every chunk of
  a prompt with only device memory changed between replays (lengths, the
  chunk's queries and mask), matches eager host-length calls bit for bit on
  every replay, with eager library work and synchronisations in between.
* The same for a whole prefill step (append + selection + attention): one
  graph replayed for every chunk of a prompt equals ChunkedPrefill.step.
"""
import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from chunked_prefill_sparse_amd.prefill import ChunkedPrefill
from oracle import chunk_attention_ref, union_tables_ref
from tests.gpu_util import (F32_MAX_ABS, Dev, check_lse, compare_bf16, oracle_full, say,
                            to_np)

pytestmark = pytest.mark.gpu


def _bern(p):
    return lambda rng, b, H, nq, pb: (rng.random((H, nq, pb)) < p).astype(np.uint8)


def _dev(vals):
    return torch.tensor([int(x) for x in vals], dtype=torch.int32, device="cuda")


CASES = [
    # B, H_q, H_kv, D, prior, chunk, C_max, dtype
    (3, 8, 2, 128, (2048, 0, 4096), (256, 192, 64), 256, "bf16"),
    (2, 6, 2, 64, (512, 1024), (128, 0), 192, "bf16"),
    (2, 4, 1, 64, (1024, 256), (256, 128), 256, "f32"),
]


@pytest.mark.parametrize("B,H_q,H_kv,D,prior,chunk,C_max,dtype", CASES)
def test_devlen_matches_host_lengths(B, H_q, H_kv, D, prior, chunk, C_max, dtype):
    w = gen.make_custom(B, H_q, H_kv, D, list(prior), list(chunk), dtype, 81, _bern(0.3),
                        C_max=C_max)
    say(f"devlen B={B} H={H_q}/{H_kv} D={D} prior={prior} chunk={chunk} {dtype}")
    d = Dev(w)
    T, lens = d.tables()
    O, lse = d.attention(T, lens, return_lse=True)
    Td, ld = ca.build_union_tables_devlen(d.mask, w.H_kv, _dev(w.n_q_blocks),
                                          _dev(w.n_kv_blocks))
    Od, lsed = ca.chunk_attention_devlen(d.q, d.k, d.v, Td, ld, _dev(w.prior), _dev(w.chunk),
                                         w.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(T, Td) and torch.equal(lens, ld)
    assert torch.equal(O, Od) and torch.equal(lse, lsed)
    Or, lr = oracle_full(w)
    if dtype == "bf16":
        compare_bf16(to_np(Od), Or, "O")
    else:
        assert np.abs(to_np(Od) - Or).max() <= F32_MAX_ABS
    check_lse(to_np(lsed), lr, fp32=dtype == "f32")


@pytest.mark.parametrize("bad", [
    dict(prior=1000),            # not a multiple of 64
    dict(chunk=320),             # past C_max
    dict(prior=-64),
    dict(prior=4096, chunk=256), # past the cache capacity L
])
def test_devlen_invalid_lengths_give_an_empty_sequence(bad):
    w = gen.make_custom(3, 8, 2, 128, [1024, 512, 2048], [256, 128, 192], "bf16", 83,
                        _bern(0.3), C_max=256)
    d = Dev(w)
    T, lens = d.tables()
    O, lse = d.attention(T, lens, return_lse=True)
    prior, chunk = list(w.prior), list(w.chunk)
    prior[1] = bad.get("prior", prior[1])
    chunk[1] = bad.get("chunk", chunk[1])
    say(f"devlen invalid lengths {bad}: sequence 1 prior {prior[1]} chunk {chunk[1]} (L {w.L})")
    Od, lsed = ca.chunk_attention_devlen(d.q, d.k, d.v, T, lens, _dev(prior), _dev(chunk),
                                         w.scale, return_lse=True)
    torch.cuda.synchronize()
    assert bool((Od[1] == 0).all()) and bool(torch.isneginf(lsed[1]).all())
    for b in (0, 2):
        assert torch.equal(Od[b], O[b]) and torch.equal(lsed[b], lse[b])


def test_devlen_union_invalid_extents_give_empty_tables():
    w = gen.make_custom(2, 8, 2, 128, [1024, 512], [256, 128], "bf16", 85, _bern(0.3),
                        with_tensors=False)
    mask = torch.from_numpy(w.mask).cuda()
    T, lens = ca.build_union_tables(mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
    nq, nkb = list(w.n_q_blocks), list(w.n_kv_blocks)
    for bad_nq, bad_nkb in ((w.NQ_max + 1, nkb[1]), (nq[1], w.NKB_max + 1), (-1, nkb[1])):
        Td, ld = ca.build_union_tables_devlen(mask, w.H_kv, _dev([nq[0], bad_nq]),
                                              _dev([nkb[0], bad_nkb]))
        torch.cuda.synchronize()
        assert torch.equal(Td[0], T[0]) and torch.equal(ld[0], lens[0])
        assert bool((ld[1] == 0).all()) and bool((Td[1] == -1).all())


def _chunk_mask(rng, H_q, C, P, NQ, NKB, p):
    """Mask of one chunk: Bernoulli prior cells, the causal block triangle, and
    ones everywhere past the chunk's extent (cells the union must ignore)."""
    m = np.ones((H_q, NQ, NKB), np.uint8)
    pblk, nq = P // 64, C // 64
    m[:, :nq, :pblk + nq] = 0
    m[:, :nq, :pblk] = rng.random((H_q, nq, pblk)) < p
    for qb in range(nq):
        m[:, qb, pblk:pblk + qb + 1] = 1
    return m


def test_one_graph_replayed_over_chunk_offsets():
    # a 2048-token prompt in 8 chunks of 256 (two sequences, the second one chunk
    # behind the first, so it starts with an empty chunk); one graph captured at
    # chunk 0, replayed for every chunk with new device lengths, queries and mask
    s = gen.make_prefill_stream("prefill_small")
    B, C, NQ, NKB = 2, s.C, s.C // 64, s.L // 64
    k = s.k.repeat(B, 1, 1, 1).cuda()
    v = s.v.repeat(B, 1, 1, 1).cuda()
    rng = np.random.default_rng(87)
    q_buf = torch.zeros((B, s.H_q, C, s.D), dtype=torch.bfloat16, device="cuda")
    mask_buf = torch.ones((B, s.H_q, NQ, NKB), dtype=torch.uint8, device="cuda")
    prior_d, chunk_d = _dev([0, 0]), _dev([0, 0])
    nq_d, nkb_d = _dev([0, 0]), _dev([0, 0])
    T = torch.empty((B, s.H_kv, NKB), dtype=torch.int32, device="cuda")
    lens = torch.empty((B, s.H_kv), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q_buf)
    lse = torch.empty((B, s.H_q, C), dtype=torch.float32, device="cuda")

    def step():
        ca.build_union_tables_devlen(mask_buf, s.H_kv, nq_d, nkb_d, T=T, lens=lens)
        ca.chunk_attention_devlen(q_buf, k, v, T, lens, prior_d, chunk_d, s.scale, out=out,
                                  lse=lse)

    def load(c):
        """Inputs of chunk c into the fixed buffers; returns the host lengths."""
        priors = [c * C, max(c - 1, 0) * C]
        chunks = [C, C if c >= 1 else 0]
        qs = [s.q_chunk(c), s.q_chunk(c - 1) if c >= 1 else torch.zeros_like(s.q_chunk(0))]
        masks = np.stack([_chunk_mask(rng, s.H_q, chunks[b], priors[b], NQ, NKB, 0.3)
                          for b in range(B)])
        q_buf.copy_(torch.cat(qs, 0))
        mask_buf.copy_(torch.from_numpy(masks))
        prior_d.copy_(_dev(priors))
        chunk_d.copy_(_dev(chunks))
        nq_d.copy_(_dev([x // 64 for x in chunks]))
        nkb_d.copy_(_dev([(p + x) // 64 for p, x in zip(priors, chunks)]))
        torch.cuda.synchronize()
        return priors, chunks, masks

    load(0)
    step()  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    k32, v32 = gen.tensor_to_f32(k.cpu()), gen.tensor_to_f32(v.cpu())
    for c in range(s.n_chunks):
        priors, chunks, masks = load(c)
        say(f"graph replay for chunk {c}: priors {priors} chunks {chunks}")
        g.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in (T, lens, out, lse)]
        # eager host-length calls on the same inputs, between replays
        Te, le = ca.build_union_tables(mask_buf, s.H_kv, [x // 64 for x in chunks],
                                       [(p + x) // 64 for p, x in zip(priors, chunks)])
        Oe, lsee = ca.chunk_attention(q_buf, k, v, Te, le, priors, chunks, s.scale,
                                      return_lse=True)
        torch.cuda.synchronize()
        for name, a, b in (("T", got[0], Te), ("lens", got[1], le), ("O", got[2], Oe),
                           ("lse", got[3], lsee)):
            assert torch.equal(a, b), f"chunk {c}: replayed {name} differs from the eager call"
        # and the oracle on the same mask bytes
        Tr, lr = union_tables_ref(masks, s.H_kv, [x // 64 for x in chunks],
                                  [(p + x) // 64 for p, x in zip(priors, chunks)])
        np.testing.assert_array_equal(got[0].cpu().numpy(), Tr)
        np.testing.assert_array_equal(got[1].cpu().numpy(), lr)
        if c in (0, 3, s.n_chunks - 1):
            q32 = gen.tensor_to_f32(q_buf.cpu())
            Or, lser = chunk_attention_ref(q32, k32, v32, Tr, lr, priors, chunks, s.scale)
            compare_bf16(to_np(got[2]), Or, f"chunk {c} O")
            check_lse(to_np(got[3]), lser, f"chunk {c} lse")
    del g


def _select_buffers(B, H_q, H_kv, NQ, NKB, D, kbar0):
    return (kbar0.clone(),
            torch.zeros((B, H_q, NQ, D), dtype=torch.float32, device="cuda"),
            torch.zeros((B, H_q, NQ, NKB), dtype=torch.float32, device="cuda"),
            torch.full((B, H_q, NQ, NKB), 7, dtype=torch.uint8, device="cuda"),
            torch.full((B, H_kv, NKB), 12345, dtype=torch.int32, device="cuda"),
            torch.full((B, H_kv), -3, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("append,D,dtype", [(False, 128, torch.bfloat16),
                                            (True, 128, torch.bfloat16),
                                            (True, 64, torch.float32)])
def test_select_devlen_matches_host_lengths(append, D, dtype):
    # ca_select_chunk_devlen / ca_append_select_chunk_devlen against the host-length
    # calls on a ragged batch, bit for bit; then sequence 1 given lengths that break
    # the limits (a chunk not a multiple of 64, a total past the cache) selects
    # nothing and appends nothing, and sequence 0 is unchanged
    B, H_kv, G, C_max, L = 3, 2, 4, 256, 4096
    H_q = H_kv * G
    prior, chunk = [3072, 1024, 0], [256, 192, 128]
    gq = torch.Generator().manual_seed(211)
    k0 = torch.randn((B, H_kv, L, D), generator=gq).to(dtype).cuda()
    v0 = torch.randn((B, H_kv, L, D), generator=gq).to(dtype).cuda()
    k_new = torch.randn((B, H_kv, C_max, D), generator=gq).to(dtype).cuda()
    v_new = torch.randn((B, H_kv, C_max, D), generator=gq).to(dtype).cuda()
    q = torch.randn((B, H_q, C_max, D), generator=gq).to(dtype).cuda()
    NQ, NKB = C_max // 64, L // 64
    kbar0 = torch.zeros((B, H_kv, NKB, D), dtype=torch.float32, device="cuda")
    ca.pool_blocks(k0, [0] * B, [p // 64 for p in prior], out=kbar0)

    def run(pr, ch):
        kc, vc = k0.clone(), v0.clone()
        bufs = _select_buffers(B, H_q, H_kv, NQ, NKB, D, kbar0)
        kbar, qbar, scores, mask, T, lens = bufs
        if append:
            ca.append_select_chunk(k_new, v_new, q, kc, vc, pr, ch, 8, 2, qbar, kbar, scores,
                                   mask, T, lens)
        else:
            ca.select_chunk(q, kc, pr, ch, 8, 2, qbar, kbar, scores, mask, T, lens)
        torch.cuda.synchronize()
        return (kc, vc) + bufs

    names = ("k_cache", "v_cache", "kbar", "qbar", "scores", "mask", "T", "lens")
    say(f"select devlen vs host lengths, append={append}, D={D}, {dtype}")
    host = run(prior, chunk)
    dev = run(_dev(prior), _dev(chunk))
    for name, a, b in zip(names, dev, host):
        assert torch.equal(a, b), name
    # sequence 1 with broken lengths: empty; sequence 0 unchanged
    for bad in ((1024, 96), (4032, 128)):
        say(f"  sequence 1 given prior {bad[0]} chunk {bad[1]}")
        pr, ch = list(prior), list(chunk)
        pr[1], ch[1] = bad
        got = run(_dev(pr), _dev(ch))
        kc, vc, kbar, qbar, scores, mask, T, lens = got
        assert int(lens[1].max()) == 0 and bool((T[1] == -1).all())
        assert bool((mask[1] == 0).all())
        assert torch.equal(kc[1], k0[1]) and torch.equal(vc[1], v0[1])
        assert torch.equal(kbar[1], kbar0[1])
        for name, a, b in zip(names, got, host):
            if name == "scores":
                nq, pb = chunk[0] // 64, prior[0] // 64
                assert torch.equal(a[0, :, :nq, :pb], b[0, :, :nq, :pb]), name
            else:
                assert torch.equal(a[0], b[0]), name


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_one_graph_serves_every_chunk(dtype):
    # ChunkedPrefill.capture_chunk: one graph of the whole step (append + selection +
    # attention, device chunk offset), captured once and replayed for every chunk of
    # prefill_small with the chunk's inputs copied into its buffers, into caches that
    # hold NaN past the appended rows; every chunk's output, mask and tables equal
    # ChunkedPrefill.step's (host offsets, resident prompt) bit for bit
    s = gen.make_prefill_stream("prefill_small")
    k_full, v_full = s.k.to(dtype).cuda(), s.v.to(dtype).cuda()
    ref = ChunkedPrefill(k_full, v_full, s.H_q, s.C, budget=4, local=2)
    qs = [s.q_chunk(c).to(dtype).cuda() for c in range(s.n_chunks)]
    priors = [c * s.C for c in range(s.n_chunks)]
    want = []
    for q, p in zip(qs, priors):
        o = ref.step(q, p).clone()
        want.append((o, ref.mask.clone(), ref.T.clone(), ref.lens.clone()))
    kc = torch.full_like(k_full, float("nan"))
    vc = torch.full_like(v_full, float("nan"))
    drv = ChunkedPrefill(kc, vc, s.H_q, s.C, budget=4, local=2)
    q_buf = torch.empty_like(qs[0])
    k_buf = torch.empty((1, s.H_kv, s.C, s.D), dtype=dtype, device="cuda")
    v_buf = torch.empty_like(k_buf)
    out = torch.empty_like(qs[0])

    def load(c):
        q_buf.copy_(qs[c])
        k_buf.copy_(k_full[:, :, priors[c]:priors[c] + s.C])
        v_buf.copy_(v_full[:, :, priors[c]:priors[c] + s.C])
        drv.set_prior(priors[c])

    # eager device-offset steps first (they also warm up before the capture)
    for c in range(s.n_chunks):
        load(c)
        drv.step_devlen(q_buf, k_buf, v_buf, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, want[c][0]), f"eager chunk {c}"
    kc.fill_(float("nan"))
    vc.fill_(float("nan"))
    g = drv.capture_chunk(q_buf, k_buf, v_buf, out=out)
    torch.cuda.synchronize()
    for rep in range(2):
        kc.fill_(float("nan"))
        vc.fill_(float("nan"))
        for c in range(s.n_chunks):
            load(c)
            say(f"one-chunk graph, {dtype}, pass {rep}, replay for chunk {c}")
            g.replay()
            torch.cuda.synchronize()
            for name, a, b in zip(("O", "mask", "T", "lens"), (out, drv.mask, drv.T, drv.lens),
                                  want[c]):
                assert torch.equal(a, b), f"pass {rep} chunk {c}: {name}"
        assert torch.equal(kc, k_full) and torch.equal(vc, v_full)
    del g
