"""GPU parity of ChunkedPrefill, the chunk-by-chunk loop (producer -> union -> attention)
over a whole prompt, against the float64 oracle chained the same way.

Each decision step is checked bit-exact in the kernel's precision (the mask
from the GPU's own scores, the tables from the GPU's mask); each floating-point
step within its bound (scores; attention over the GPU's tables).  The dense
baseline of ChunkedPrefill is checked on every chunk too.
"""
import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from chunked_prefill_sparse_amd.prefill import ChunkedPrefill
from oracle import (block_scores_ref, chunk_attention_ref, chunk_attention_rows_ref,
                    pool_blocks_ref, topk_mask_ref, union_tables_ref)
from tests.gpu_util import check_lse, check_scores, compare_bf16, say, score_bound, to_np

pytestmark = pytest.mark.gpu



@pytest.mark.parametrize("balanced", [False, True])
def test_prefill_small_every_chunk(balanced):
    s = gen.make_prefill_stream("prefill_small")
    k_dev, v_dev = s.k.cuda(), s.v.cuda()
    drv = ChunkedPrefill(k_dev, v_dev, s.H_q, s.C, budget=4, local=2, balanced=balanced)
    k, v = gen.tensor_to_f32(s.k), gen.tensor_to_f32(s.v)
    kr = np.nan_to_num(pool_blocks_ref(k, [0], [s.L // 64], s.L // 64))
    for c in range(s.n_chunks):
        P = c * s.C
        say(f"prefill_small chunk {c} prior {P} balanced={balanced}")
        q_cpu = s.q_chunk(c)
        q_dev = q_cpu.cuda()
        O = drv.step(q_dev, P).clone()
        Od = drv.step_dense(q_dev, P, drv.dense_lens(P)).clone()
        torch.cuda.synchronize()
        q = gen.tensor_to_f32(q_cpu)
        nq, pblk, nkb = s.C // 64, P // 64, (P + s.C) // 64
        # scores (floating point) against the float64 pooled scores
        qr = pool_blocks_ref(q, [0], [nq], nq)
        sr = block_scores_ref(qr, kr)
        sg = drv.scores.cpu().numpy().astype(np.float64)
        check_scores(sg[..., :pblk], sr[..., :pblk], score_bound(qr, kr)[..., :pblk])
        # mask: bit-exact from the GPU's own scores
        sel_in = np.zeros_like(sg)
        sel_in[..., :pblk] = sg[..., :pblk]
        m = drv.mask.cpu().numpy()
        np.testing.assert_array_equal(m, topk_mask_ref(sel_in, [P], [s.C], 4, 2, s.L // 64))
        # tables: bit-exact from the GPU's mask
        T, ln = union_tables_ref(m, s.H_kv, [nq], [nkb])
        np.testing.assert_array_equal(drv.T.cpu().numpy(), T)
        np.testing.assert_array_equal(drv.lens.cpu().numpy(), ln)
        # attention over those tables, and the dense baseline
        Or, _ = chunk_attention_ref(q, k, v, T, ln, [P], [s.C], s.scale)
        compare_bf16(to_np(O), Or, f"chunk {c} sparse")
        Td = np.broadcast_to(np.arange(s.L // 64, dtype=np.int32), (1, s.H_kv, s.L // 64))
        Odr, _ = chunk_attention_ref(q, k, v, np.ascontiguousarray(Td),
                                     np.full((1, s.H_kv), nkb, np.int32), [P], [s.C], s.scale)
        compare_bf16(to_np(Od), Odr, f"chunk {c} dense")
        if pblk > 8:
            # the planted salient blocks are found by every row once they fit the budget
            sal = s.salient_blocks
            for g in range(s.H_kv):
                found = set(T[0, g, :ln[0, g]].tolist())
                want = set(np.flatnonzero(sal[g, :pblk]).tolist())
                if len(want) <= 4:
                    assert want <= found, (c, g, want - found)


@pytest.mark.parametrize("balanced", [False, True])
def test_prefill_graph_replay_matches_eager(balanced):
    # The whole prompt (select + attend per chunk, and the dense baseline)
    # recorded into one HIP graph: every replay, with eager library work and
    # synchronisations in between, reproduces the eager outputs bit for bit.
    s = gen.make_prefill_stream("prefill_small")
    k_dev, v_dev = s.k.cuda(), s.v.cuda()
    drv = ChunkedPrefill(k_dev, v_dev, s.H_q, s.C, budget=4, local=2, balanced=balanced)
    qs = [s.q_chunk(c).cuda() for c in range(s.n_chunks)]
    priors = [c * s.C for c in range(s.n_chunks)]
    eager = [drv.step(q, p).clone() for q, p in zip(qs, priors)]
    eager_T, eager_lens = drv.T.clone(), drv.lens.clone()
    eager_d = [drv.step_dense(q, p, drv.dense_lens(p)).clone() for q, p in zip(qs, priors)]
    torch.cuda.synchronize()
    outs = [torch.full_like(qs[0], float("nan")) for _ in qs]
    outs_d = [torch.full_like(qs[0], float("nan")) for _ in qs]
    g = drv.capture(qs, priors, outs=outs)
    gd = drv.capture(qs, priors, outs=outs_d, dense=True)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"graph replay {rep}")
        for o in outs + outs_d:
            o.fill_(float("nan"))
        drv.step(qs[0], 0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        gd.replay()
        torch.cuda.synchronize()
        for c in range(s.n_chunks):
            assert torch.equal(outs[c], eager[c]), (rep, c)
            assert torch.equal(outs_d[c], eager_d[c]), (rep, c)
        assert torch.equal(drv.T, eager_T) and torch.equal(drv.lens, eager_lens)


@pytest.mark.parametrize("balanced,fused", [(False, True), (True, True), (False, False)])
def test_prefill_overlap_matches_sequential(balanced, fused):
    # run(overlap=True): each chunk's append and selection on a second stream, one
    # chunk ahead of the attention, into caches that hold NaN past the appended rows.
    # Every chunk's output equals the sequential steps' over the resident prompt, bit
    # for bit, eagerly and from a graph of the two streams replayed three times with
    # eager work in between; the caches end up equal to the prompt.
    s = gen.make_prefill_stream("prefill_small")
    k_full, v_full = s.k.cuda(), s.v.cuda()
    ref = ChunkedPrefill(k_full, v_full, s.H_q, s.C, budget=4, local=2)
    qs = [s.q_chunk(c).cuda() for c in range(s.n_chunks)]
    priors = [c * s.C for c in range(s.n_chunks)]
    want = [ref.step(q, p).clone() for q, p in zip(qs, priors)]
    kv = [(k_full[:, :, p:p + s.C].contiguous(), v_full[:, :, p:p + s.C].contiguous())
          for p in priors]
    kc = torch.full_like(k_full, float("nan"))
    vc = torch.full_like(v_full, float("nan"))
    drv = ChunkedPrefill(kc, vc, s.H_q, s.C, budget=4, local=2, balanced=balanced,
                         fused_append=fused)
    outs = [torch.full_like(qs[0], float("nan")) for _ in qs]
    torch.cuda.synchronize()
    say(f"overlapped prefill_small, eager, balanced={balanced}, fused append={fused}")
    drv.run(qs, priors, outs=outs, kv_chunks=kv, overlap=True)
    torch.cuda.synchronize()
    for c in range(s.n_chunks):
        assert torch.equal(outs[c], want[c]), c
    last = drv.tables[(s.n_chunks - 1) % len(drv.tables)]
    assert torch.equal(last[0], ref.T) and torch.equal(last[1], ref.lens)
    assert torch.equal(kc, k_full) and torch.equal(vc, v_full)
    kc.fill_(float("nan"))
    vc.fill_(float("nan"))
    g = drv.capture(qs, priors, outs=outs, kv_chunks=kv, overlap=True)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"overlapped graph replay {rep}")
        for o in outs:
            o.fill_(float("nan"))
        kc.fill_(float("nan"))
        vc.fill_(float("nan"))
        drv.run(qs[:1], priors[:1], kv_chunks=kv[:1], overlap=False)  # eager work between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for c in range(s.n_chunks):
            assert torch.equal(outs[c], want[c]), (rep, c)
        assert torch.equal(kc, k_full) and torch.equal(vc, v_full)


def test_prefill_small_append_from_poisoned_cache():
    # Each chunk's keys and values are appended at its step into caches that hold
    # NaN everywhere else: every chunk's mask, tables and outputs (sparse and dense)
    # equal those of the run over the resident prompt, bit for bit, so nothing
    # reads a cache row before its chunk has been appended.
    s = gen.make_prefill_stream("prefill_small")
    k_full, v_full = s.k.cuda(), s.v.cuda()
    ref = ChunkedPrefill(k_full, v_full, s.H_q, s.C, budget=4, local=2)
    kc = torch.full_like(k_full, float("nan"))
    vc = torch.full_like(v_full, float("nan"))
    drv = ChunkedPrefill(kc, vc, s.H_q, s.C, budget=4, local=2)
    for c in range(s.n_chunks):
        P = c * s.C
        q = s.q_chunk(c).cuda()
        kch = k_full[:, :, P:P + s.C].contiguous()
        vch = v_full[:, :, P:P + s.C].contiguous()
        O_ref = ref.step(q, P).clone()
        O = drv.step(q, P, k_chunk=kch, v_chunk=vch).clone()
        torch.cuda.synchronize()
        say(f"prefill_small with append, chunk {c}")
        assert torch.equal(drv.mask, ref.mask) and torch.equal(drv.T, ref.T)
        assert torch.equal(drv.lens, ref.lens) and torch.equal(O, O_ref)
        Od_ref = ref.step_dense(q, P, ref.dense_lens(P)).clone()
        Od = drv.step_dense(q, P, drv.dense_lens(P)).clone()
        torch.cuda.synchronize()
        assert torch.equal(Od, Od_ref)
    assert torch.equal(kc, k_full) and torch.equal(vc, v_full)


def test_prefill_128k_sampled_chunks():
    # The 128K prompt (64 chunks of 2048, LLaMA-8B attention shape) through the
    # whole chunk loop with append, from NaN-poisoned caches.  At chunks 0, 31
    # and 63 the chain is checked against the oracle as for prefill_small: scores
    # against float64, the mask bit-exact from the GPU's scores, the tables
    # bit-exact from the GPU's mask, and attention (O and lse) on sampled rows of
    # every KV group over those tables.
    s = gen.make_prefill_stream("prefill_128k")
    budget, local = 32, 8
    k_full, v_full = s.k.cuda(), s.v.cuda()
    kc = torch.full_like(k_full, float("nan"))
    vc = torch.full_like(v_full, float("nan"))
    drv = ChunkedPrefill(kc, vc, s.H_q, s.C, budget=budget, local=local)
    k32, v32 = gen.tensor_to_f32(s.k), gen.tensor_to_f32(s.v)
    kr = np.nan_to_num(pool_blocks_ref(k32, [0], [s.L // 64], s.L // 64))
    rng = np.random.default_rng(1006)
    for c in range(s.n_chunks):
        P = c * s.C
        q_cpu = s.q_chunk(c)
        q_dev = q_cpu.cuda()
        O = drv.step(q_dev, P, k_chunk=k_full[:, :, P:P + s.C].contiguous(),
                     v_chunk=v_full[:, :, P:P + s.C].contiguous())
        if c not in (0, 31, s.n_chunks - 1):
            continue
        O2, lse = ca.chunk_attention(q_dev, drv.k, drv.v, drv.T, drv.lens, [P], [s.C], s.scale,
                                     return_lse=True)
        torch.cuda.synchronize()
        say(f"prefill_128k chunk {c} prior {P}: checking against the oracle")
        assert torch.equal(O, O2) and bool(torch.isfinite(O).all())
        q = gen.tensor_to_f32(q_cpu)
        nq, pblk, nkb = s.C // 64, P // 64, (P + s.C) // 64
        sg = drv.scores.cpu().numpy().astype(np.float64)
        if pblk:
            qr = pool_blocks_ref(q, [0], [nq], nq)
            sr = block_scores_ref(qr, kr)
            check_scores(sg[..., :pblk], sr[..., :pblk], score_bound(qr, kr)[..., :pblk])
        sel_in = np.zeros_like(sg)
        sel_in[..., :pblk] = sg[..., :pblk]
        m = drv.mask.cpu().numpy()
        np.testing.assert_array_equal(m, topk_mask_ref(sel_in, [P], [s.C], budget, local,
                                                       s.L // 64))
        T, ln = union_tables_ref(m, s.H_kv, [nq], [nkb])
        np.testing.assert_array_equal(drv.T.cpu().numpy(), T)
        np.testing.assert_array_equal(drv.lens.cpu().numpy(), ln)
        say(f"  union blocks {int(ln.sum())} of {s.H_kv * nkb}")
        rows = []
        for g in range(s.H_kv):
            for h in rng.choice(np.arange(g * s.G, (g + 1) * s.G), size=2, replace=False):
                for i in [0, 1, 31, 32, 63, 64, 1023, 1024, 2015, 2016, 2046, 2047] + \
                        [int(x) for x in rng.integers(0, s.C, 4)]:
                    rows.append((0, int(h), i))
        rows = np.array(sorted(set(rows)), np.int64)
        Or, lr = chunk_attention_rows_ref(q, k32, v32, T, ln, [P], [s.C], s.scale, rows)
        r = torch.from_numpy(rows).cuda()
        compare_bf16(to_np(O[r[:, 0], r[:, 1], r[:, 2]]), Or, f"chunk {c}, {len(rows)} rows")
        check_lse(to_np(lse[r[:, 0], r[:, 1], r[:, 2]]), lr, f"chunk {c} lse")
