"""Pins for the block-mask producer oracle (CPU only).

The pages leave the pattern searcher open; the producer here is defined by
its own docstring (pooled scores, per-row top-k, forced sink / local window /
causal block triangle).  Pinned by closed forms of the pooling (constant and
linear rows), a pure-Python brute force of the scores, a lexsort brute force
of the selection with planted ties, invariants (count, monotone in the
budget, forced cells, empty rows beyond the chunk) and a planted-signal case
where the right blocks must win.
"""
import numpy as np
import pytest

from oracle import block_scores_ref, pool_blocks_ref, producer_mask_ref, topk_mask_ref


def test_pool_closed_forms():
    B, H, R, D = 2, 3, 5 * 64, 4
    x = np.zeros((B, H, R, D), np.float32)
    x[..., 0] = 2.5                                   # constant column
    x[..., 1] = np.arange(R, dtype=np.float32)        # linear rows
    out = pool_blocks_ref(x, [1, 0], [4, 2], 6)
    for b, (lo, hi) in enumerate([(1, 4), (0, 2)]):
        for kb in range(6):
            if lo <= kb < hi:
                assert out[b, 0, kb, 0] == 2.5
                assert out[b, 2, kb, 1] == 64 * kb + 31.5
                assert out[b, 1, kb, 2] == 0.0
            else:
                assert np.isnan(out[b, :, kb]).all()


def test_scores_brute_force():
    rng = np.random.default_rng(0)
    qbar = rng.standard_normal((1, 4, 3, 5))
    kbar = rng.standard_normal((1, 2, 7, 5))
    s = block_scores_ref(qbar, kbar)
    for h in range(4):
        for qb in range(3):
            for kb in range(7):
                ref = sum(qbar[0, h, qb, d] * kbar[0, h // 2, kb, d] for d in range(5))
                assert abs(s[0, h, qb, kb] - ref) < 1e-12


def _brute_select(s_row, cand, budget):
    # lexsort: primary key -score, secondary kb
    order = np.lexsort((cand, -s_row[cand]))
    return set(cand[order[:budget]].tolist())


@pytest.mark.parametrize("budget,local", [(0, 4), (5, 4), (10, 0), (40, 2), (200, 8)])
def test_selection_brute_force(budget, local):
    rng = np.random.default_rng(budget + 17 * local)
    B, H, NQ, NKB = 2, 3, 4, 64
    prior, chunk = [40 * 64, 3 * 64], [4 * 64, 2 * 64]
    s = np.round(rng.standard_normal((B, H, NQ, NKB)), 1)  # rounding plants many ties
    m = topk_mask_ref(s, prior, chunk, budget, local, NKB)
    for b in range(B):
        P, nq = prior[b] // 64, chunk[b] // 64
        lo = max(P - local, 1)
        cand = np.arange(1, lo)
        for h in range(H):
            for qb in range(NQ):
                row = m[b, h, qb]
                if qb >= nq:
                    assert not row.any()
                    continue
                forced = ({0} if P else set()) | set(range(lo, P)) | set(range(P, P + qb + 1))
                chosen = _brute_select(s[b, h, qb], cand, budget) if cand.size else set()
                assert set(np.flatnonzero(row).tolist()) == forced | chosen
                assert len(chosen) == min(budget, cand.size)


def test_selection_monotone_in_budget():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((1, 2, 2, 100))
    prev = None
    for budget in (0, 1, 3, 10, 50, 95, 200):
        m = topk_mask_ref(s, [90 * 64], [2 * 64], budget, 3, 100)
        if prev is not None:
            assert ((m >= prev)).all()
        prev = m


def test_planted_blocks_win():
    rng = np.random.default_rng(11)
    B, H_q, H_kv, D, P, C = 1, 4, 2, 32, 50 * 64, 2 * 64
    q = rng.standard_normal((B, H_q, C, D)).astype(np.float32)
    k = rng.standard_normal((B, H_kv, P + C, D)).astype(np.float32)
    u = rng.standard_normal((H_kv, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    planted = {0: [5, 17, 33], 1: [2, 20, 41]}
    for g, blocks in planted.items():
        for kb in blocks:
            k[0, g, kb * 64:(kb + 1) * 64] += 4 * u[g]
        q[0, 2 * g:2 * g + 2] += 4 * u[g]
    m = producer_mask_ref(q, k, [P], [C], budget=3, local=2, NKB_max=P // 64 + 2)
    for h in range(H_q):
        for qb in range(2):
            sel = set(np.flatnonzero(m[0, h, qb, 1:P // 64 - 2]) + 1)
            assert sel == set(planted[h // 2])
