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
from chunked_prefill_sparse_amd.prefill import ChunkedPrefill
from oracle import (block_scores_ref, chunk_attention_ref, pool_blocks_ref, topk_mask_ref,
                    union_tables_ref)
from tests.gpu_util import compare_bf16, say, to_np

pytestmark = pytest.mark.gpu

SCORE_ATOL = 2e-5


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
        np.testing.assert_allclose(sg[..., :pblk], sr[..., :pblk], rtol=0, atol=SCORE_ATOL)
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
