"""Pins for the compaction oracle (CPU only).

CompactAttention, abstract: the tables let attention read selected blocks in
place instead of compacting them.  The compaction baseline must therefore
leave the attention result unchanged; that invariant, a hand-worked case and
structural checks (contiguity, chunk blocks untouched) pin the oracle.
"""
import numpy as np
import pytest

import gen
from oracle import chunk_attention_ref, compact_kv_ref, union_tables_ref


def test_hand_worked_case():
    # prior = 5 blocks, chunk = 2 blocks; table selects prior blocks 0, 3 and
    # chunk blocks 5, 6.  p = 2 prior entries land on blocks 3, 4 (ending where
    # the chunk starts, block 5); chunk blocks stay at 5, 6.
    L, D = 8 * 64, 4
    k = np.arange(1 * 1 * L * D, dtype=np.float32).reshape(1, 1, L, D)
    v = -k
    T = np.array([[[0, 3, 5, 6, -1, -1, -1, -1]]], np.int32)
    ln = np.array([[4]], np.int32)
    k_out, v_out, T_out, written = compact_kv_ref(k, v, T, ln, [5 * 64], [2 * 64])
    assert T_out.tolist() == [[[3, 4, 5, 6, -1, -1, -1, -1]]]
    assert written[0, 0].tolist() == [False, False, False, True, True, True, True, False]
    blk = lambda a, i: a[0, 0, i * 64:(i + 1) * 64]  # noqa: E731
    np.testing.assert_array_equal(blk(k_out, 3), blk(k, 0))
    np.testing.assert_array_equal(blk(k_out, 4), blk(k, 3))
    np.testing.assert_array_equal(blk(k_out, 5), blk(k, 5))
    np.testing.assert_array_equal(blk(v_out, 6), blk(v, 6))
    assert not k_out[0, 0, :3 * 64].any()


def test_empty_and_prior_only_tables():
    L, D = 4 * 64, 2
    k = np.ones((1, 2, L, D), np.float32)
    T = np.array([[[-1, -1, -1, -1], [0, 1, -1, -1]]], np.int32)
    ln = np.array([[0, 2]], np.int32)
    _, _, T_out, written = compact_kv_ref(k, k, T, ln, [4 * 64], [0])
    assert T_out[0, 0].tolist() == [-1, -1, -1, -1]
    assert T_out[0, 1].tolist() == [2, 3, -1, -1]
    assert not written[0, 0].any() and written[0, 1].tolist() == [False, False, True, True]


@pytest.mark.parametrize("seed,dtype", [(11, "f32"), (12, "bf16"), (13, "f32")])
def test_attention_unchanged_by_compaction(seed, dtype):
    rng = np.random.default_rng(seed)
    w = gen.make_custom(B=2, H_q=4, H_kv=2, D=16, prior=[640, 384], chunk=[192, 128],
                        dtype=dtype, seed=seed,
                        cell_fn=lambda r, b, H, nq, pb: (r.random((H, nq, pb)) < 0.3).astype(np.uint8))
    T, ln = union_tables_ref(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
    q, k, v = (gen.tensor_to_f32(x) for x in (w.q, w.k, w.v))
    O0, l0 = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    k2, v2, T2, written = compact_kv_ref(k, v, T, ln, w.prior, w.chunk)
    # poison every block the compaction did not write: none of it may be read
    blocks = k2.reshape(w.B, w.H_kv, -1, 64, w.D)
    blocks[~written] = rng.standard_normal(blocks[~written].shape) * 1e3
    O1, l1 = chunk_attention_ref(q, k2, v2, T2, ln, w.prior, w.chunk, w.scale)
    np.testing.assert_array_equal(O0, O1)
    np.testing.assert_array_equal(l0, l1)
    for b in range(w.B):
        P_blk = w.prior[b] // 64
        for g in range(w.H_kv):
            t = T2[b, g, :ln[b, g]]
            prior_part = t[t < P_blk]
            # packed: a contiguous run that ends at the chunk's first block
            assert prior_part.tolist() == list(range(P_blk - prior_part.size, P_blk))
            chunk_part = T[b, g, :ln[b, g]][T[b, g, :ln[b, g]] >= P_blk]
            assert t[t >= P_blk].tolist() == chunk_part.tolist()
