"""Pins for the block-sparse-execution oracle (CPU only).

The pages define the baseline only in words (the 2D mask used directly as a
sparse kernel's execution plan: each Q-block of each head attends its own
mask row).  It is pinned here by pure-Python brute force with math.exp, by
its reduction to the union attention when every mask row of a group is the
group's union (rows widened to the union, or masks constant over Q-blocks and
heads), by the dense special case, and by the sampled-row form agreeing with
the full one.
"""
import math

import numpy as np
import pytest

import gen
from oracle import (chunk_attention_ref, sparse_attention_ref, sparse_attention_rows_ref,
                    union_tables_ref)


def _w(seed, p=0.3, B=2, H_q=4, H_kv=2, D=16, prior=(320, 192), chunk=(192, 128), **kw):
    return gen.make_custom(B, H_q, H_kv, D, list(prior), list(chunk), "f32", seed,
                           lambda rng, b, H, nq, pb: (rng.random((H, nq, pb)) < p).astype(np.uint8),
                           **kw)


def _arrays(w):
    return gen.tensor_to_f32(w.q), gen.tensor_to_f32(w.k), gen.tensor_to_f32(w.v)


def test_brute_force_tiny():
    w = _w(3, B=1, H_q=2, H_kv=1, D=4, prior=(128,), chunk=(128,))
    q, k, v = _arrays(w)
    O, lse = sparse_attention_ref(q, k, v, w.mask, w.prior, w.chunk, w.scale)
    P, C = w.prior[0], w.chunk[0]
    for h in range(2):
        for i in range(C):
            p = P + i
            xs, vs = [], []
            for t in range(P + C):
                if t <= p and w.mask[0, h, i // 64, t // 64]:
                    xs.append(w.scale * sum(float(q[0, h, i, d]) * float(k[0, 0, t, d])
                                            for d in range(4)))
                    vs.append([float(x) for x in v[0, 0, t]])
            m = max(xs)
            e = [math.exp(x - m) for x in xs]
            s = sum(e)
            ref = [sum(e[n] * vs[n][d] for n in range(len(e))) / s for d in range(4)]
            np.testing.assert_allclose(O[0, h, i], ref, rtol=1e-6, atol=1e-7)
            assert abs(lse[0, h, i] - (m + math.log(s))) < 1e-5


@pytest.mark.parametrize("seed", [1, 2])
def test_rows_widened_to_the_union_give_union_attention(seed):
    w = _w(seed)
    q, k, v = _arrays(w)
    T, ln = union_tables_ref(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
    wide = np.zeros_like(w.mask)
    for b in range(w.B):
        for g in range(w.H_kv):
            wide[b, g * w.G:(g + 1) * w.G, :, T[b, g, :ln[b, g]]] = 1
    Os, ls = sparse_attention_ref(q, k, v, wide, w.prior, w.chunk, w.scale)
    Ou, lu = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    np.testing.assert_allclose(Os, Ou, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(ls, lu, rtol=1e-6, atol=1e-6)


def test_rows_differ_from_union_when_masks_differ():
    # a mask that differs across Q-blocks: the sparse result must not be the union's
    w = _w(5, p=0.2)
    q, k, v = _arrays(w)
    T, ln = union_tables_ref(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
    Os, _ = sparse_attention_ref(q, k, v, w.mask, w.prior, w.chunk, w.scale)
    Ou, _ = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    assert np.abs(Os - Ou).max() > 1e-3


def test_dense_mask_equals_dense_attention():
    w = _w(7, p=1.0)
    q, k, v = _arrays(w)
    nkb = max(w.n_kv_blocks)
    T = np.broadcast_to(np.arange(w.mask.shape[3], dtype=np.int32), (w.B, w.H_kv, w.mask.shape[3]))
    ln = np.array([[n] * w.H_kv for n in w.n_kv_blocks], np.int32)
    assert nkb <= w.mask.shape[3]
    Os, ls = sparse_attention_ref(q, k, v, np.ones_like(w.mask), w.prior, w.chunk, w.scale)
    Ou, lu = chunk_attention_ref(q, k, v, np.ascontiguousarray(T), ln, w.prior, w.chunk, w.scale)
    np.testing.assert_allclose(Os, Ou, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(ls, lu, rtol=1e-6, atol=1e-6)


def test_sampled_rows_match_full():
    w = _w(9)
    q, k, v = _arrays(w)
    O, lse = sparse_attention_ref(q, k, v, w.mask, w.prior, w.chunk, w.scale)
    rows = np.array([(b, h, i) for b in range(w.B) for h in range(w.H_q)
                     for i in (0, 1, 63, 64, 100, w.chunk[b] - 1, w.C_max - 1)], np.int64)
    Or, lr = sparse_attention_rows_ref(q, k, v, w.mask, w.prior, w.chunk, w.scale, rows)
    np.testing.assert_allclose(Or, O[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=1e-6, atol=1e-7)
    np.testing.assert_array_equal(np.isinf(lr), np.isinf(lse[rows[:, 0], rows[:, 1], rows[:, 2]]))
