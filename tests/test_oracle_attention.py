"""Pins for the chunk-attention oracle (CPU only).

The pages fix the dense special case (the same execution fed every block is
the dense attention baseline the speedups are measured against) and that only
the selected blocks are read.  The oracle is pinned here against torch's
scaled_dot_product_attention (float64, CPU, explicit boolean mask) on the
dense case, a pure-Python brute force with math.exp on tiny inputs, closed
forms (K = 0, one-hot V, V = 1, a single admissible key), shift invariance of
the softmax, the empty-set convention, and poison invariance.
"""
import math

import numpy as np
import pytest
import torch

import gen
from oracle import (admissible_keys, chunk_attention_dense_masked_ref, chunk_attention_ref,
                    chunk_attention_rows_ref, union_tables_ref)


def _arrays(w):
    return gen.tensor_to_f32(w.q), gen.tensor_to_f32(w.k), gen.tensor_to_f32(w.v)


def _tables(w):
    return union_tables_ref(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)


def _tiny(B=2, H_q=4, H_kv=2, D=16, prior=(128, 192), chunk=(128, 64), p=0.4, seed=0,
          triangle=True, **kw):
    return gen.make_custom(B, H_q, H_kv, D, list(prior), list(chunk), "f32", seed,
                           lambda rng, b, H, nq, pb: (rng.random((H, nq, pb)) < p).astype(np.uint8),
                           triangle=triangle, **kw)


def _sdpa_dense_causal(q, k, v, prior, chunk, scale):
    """torch SDPA in float64 with an explicit boolean mask: query row i of the
    chunk (absolute position prior+i) sees cached keys t <= prior+i."""
    B, H_q, C_max, D = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    out = np.zeros_like(q, dtype=np.float64)
    for b in range(B):
        P, C = prior[b], chunk[b]
        n = P + C
        qt = torch.from_numpy(q[b, :, :C].astype(np.float64))
        kt = torch.from_numpy(np.repeat(k[b, :, :n], G, axis=0).astype(np.float64))
        vt = torch.from_numpy(np.repeat(v[b, :, :n], G, axis=0).astype(np.float64))
        allowed = torch.arange(n)[None, :] <= (P + torch.arange(C))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed,
                                                             scale=scale)
        out[b, :, :C] = o.numpy()
    return out


@pytest.mark.parametrize("B,H_q,H_kv,D,prior,chunk", [
    (1, 4, 1, 64, (1024,), (256,)),
    (2, 8, 2, 32, (256, 640), (128, 192)),
    (2, 4, 4, 16, (0, 64), (64, 128)),
])
def test_dense_case_matches_sdpa(B, H_q, H_kv, D, prior, chunk):
    w = gen.make_custom(B, H_q, H_kv, D, list(prior), list(chunk), "f32", 42,
                        lambda rng, b, H, nq, pb: np.ones((H, nq, pb), np.uint8))
    w.mask[:] = 1
    q, k, v = _arrays(w)
    T, ln = _tables(w)
    O, _ = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    ref = _sdpa_dense_causal(q, k, v, w.prior, w.chunk, w.scale)
    np.testing.assert_allclose(O, ref, rtol=0, atol=2e-6)


def test_tiny_f32_workload_dense_variant_matches_sdpa():
    w = gen.make_workload("tiny_f32")
    w.mask[:] = 1
    q, k, v = _arrays(w)
    T, ln = _tables(w)
    O, _ = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    ref = _sdpa_dense_causal(q, k, v, w.prior, w.chunk, w.scale)
    np.testing.assert_allclose(O, ref, rtol=0, atol=2e-6)


def _brute(q, k, v, T, ln, prior, chunk, scale):
    """One (b, h, i) at a time with Python loops and math.exp."""
    B, H_q, C_max, D = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    O = np.zeros((B, H_q, C_max, D))
    lse = np.full((B, H_q, C_max), -np.inf)
    for b in range(B):
        for h in range(H_q):
            g = h // G
            blocks = set(int(x) for x in T[b, g, :ln[b, g]])
            for i in range(chunk[b]):
                p = prior[b] + i
                xs = []
                for t in range(prior[b] + chunk[b]):
                    if t // 64 in blocks and t <= p:
                        xs.append((t, scale * sum(float(q[b, h, i, d]) * float(k[b, g, t, d])
                                                  for d in range(D))))
                if not xs:
                    continue
                mx = max(x for _, x in xs)
                ws = [(t, math.exp(x - mx)) for t, x in xs]
                s = sum(wt for _, wt in ws)
                for d in range(D):
                    O[b, h, i, d] = sum(wt * float(v[b, g, t, d]) for t, wt in ws) / s
                lse[b, h, i] = mx + math.log(s)
    return O, lse


@pytest.mark.parametrize("prior,chunk,triangle", [
    ((128, 64), (70, 64), True),    # unaligned chunk length
    ((100, 64), (40, 33), True),    # unaligned prior
    ((128, 192), (64, 64), False),  # no current-chunk blocks forced: empty rows possible
])
def test_brute_force(prior, chunk, triangle):
    w = _tiny(B=2, H_q=4, H_kv=2, D=4, prior=prior, chunk=chunk, p=0.35, seed=3,
              triangle=triangle)
    q, k, v = _arrays(w)
    T, ln = _tables(w)
    O, lse = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    Ob, lseb = _brute(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-6)
    np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-5)


def test_second_formulation_agrees():
    for seed in range(4):
        w = _tiny(seed=seed, prior=(256, 320), chunk=(192, 128), p=0.3)
        q, k, v = _arrays(w)
        T, ln = _tables(w)
        O1, l1 = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
        O2, l2 = chunk_attention_dense_masked_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
        np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-6)
        np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-5)


def test_rows_oracle_matches_full():
    w = _tiny(seed=5, prior=(256, 128), chunk=(128, 96), C_max=128)
    q, k, v = _arrays(w)
    T, ln = _tables(w)
    O, lse = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    rng = np.random.default_rng(0)
    rows = np.stack([rng.integers(0, 2, 40), rng.integers(0, 4, 40), rng.integers(0, 128, 40)], 1)
    Or, lr = chunk_attention_rows_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale, rows)
    np.testing.assert_array_equal(Or, O[rows[:, 0], rows[:, 1], rows[:, 2]])
    np.testing.assert_array_equal(lr, lse[rows[:, 0], rows[:, 1], rows[:, 2]])


def _count_admissible(T, ln, b, g, P, C, i):
    return admissible_keys(T[b, g], int(ln[b, g]), P, C, P + i).size


def test_closed_form_zero_keys_gives_mean_of_values():
    w = _tiny(seed=8, D=16, p=0.3)
    q, k, v = _arrays(w)
    k[:] = 0.0
    T, ln = _tables(w)
    O, lse = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    G = w.G
    for b in range(w.B):
        P, C = w.prior[b], w.chunk[b]
        for h in range(w.H_q):
            g = h // G
            for i in range(C):
                keys = admissible_keys(T[b, g], int(ln[b, g]), P, C, P + i)
                np.testing.assert_allclose(O[b, h, i], v[b, g, keys].astype(np.float64).mean(0),
                                           rtol=0, atol=1e-6)
                assert abs(lse[b, h, i] - math.log(keys.size)) < 1e-6


def test_closed_form_one_hot_values_show_blocks_read():
    # D >= number of blocks: V_t = one_hot(t // 64), K = 0.  Then O[., kb] is the
    # share of admissible keys that lie in block kb; zero for blocks not in T.
    w = gen.make_workload("tiny_f32")  # 20 blocks, D = 64
    q, k, v = _arrays(w)
    k[:] = 0.0
    v[:] = 0.0
    n_tok = w.prior[0] + w.chunk[0]
    v[0, 0, np.arange(n_tok), np.arange(n_tok) // 64] = 1.0
    T, ln = _tables(w)
    O, _ = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    sel = set(T[0, 0, :ln[0, 0]].tolist())
    P = w.prior[0]
    for h in range(w.H_q):
        for i in range(w.chunk[0]):
            keys = admissible_keys(T[0, 0], int(ln[0, 0]), P, w.chunk[0], P + i)
            expect = np.bincount(keys // 64, minlength=64) / keys.size
            np.testing.assert_allclose(O[0, h, i], expect, rtol=0, atol=1e-7)
            assert all(O[0, h, i, kb] == 0.0 for kb in range(20) if kb not in sel)
            # causal: nothing beyond the row's own position
            assert O[0, h, i, (P + i) // 64 + 1:].sum() == 0.0


def test_closed_form_constant_values():
    w = _tiny(seed=9)
    q, k, v = _arrays(w)
    v[:] = 1.0
    T, ln = _tables(w)
    O, _ = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    for b in range(w.B):
        np.testing.assert_allclose(O[b, :, :w.chunk[b]], 1.0, rtol=0, atol=1e-12)


def test_single_admissible_key_returns_its_value():
    # No prior block selected (no sink, no triangle for the prior part): row 0 of the
    # chunk sees exactly its own key, so O = V[prior] exactly.
    w = _tiny(B=1, H_q=2, H_kv=1, prior=(128,), chunk=(64,), p=0.0, seed=2)
    q, k, v = _arrays(w)
    T, ln = _tables(w)
    assert T[0, 0, :ln[0, 0]].tolist() == [2]
    O, lse = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    for h in range(2):
        np.testing.assert_array_equal(O[0, h, 0], v[0, 0, 128])
        assert abs(lse[0, h, 0] - w.scale * float(q[0, h, 0] @ k[0, 0, 128].astype(np.float64))) < 1e-6


def test_empty_admissible_set_and_padding_rows():
    w = _tiny(B=1, H_q=2, H_kv=1, prior=(128,), chunk=(64,), p=0.0, seed=2, triangle=False,
              C_max=96)
    q, k, v = _arrays(w)
    T, ln = _tables(w)
    assert ln[0, 0] == 0
    O, lse = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    assert np.all(O == 0) and np.all(np.isneginf(lse))
    w2 = _tiny(B=1, H_q=2, H_kv=1, prior=(128,), chunk=(64,), p=0.5, seed=2, C_max=96)
    q, k, v = _arrays(w2)
    T, ln = _tables(w2)
    O, lse = chunk_attention_ref(q, k, v, T, ln, w2.prior, w2.chunk, w2.scale)
    assert np.all(O[0, :, 64:] == 0) and np.all(np.isneginf(lse[0, :, 64:]))
    assert np.all(np.isfinite(lse[0, :, :64]))


def test_shift_invariance_of_keys():
    # Adding one vector u to every key shifts each row's logits by the same amount:
    # O is unchanged and LSE moves by scale * q.u.
    w = _tiny(seed=12, D=8)
    q, k, v = _arrays(w)
    T, ln = _tables(w)
    O, lse = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    u = np.random.default_rng(1).standard_normal(w.D).astype(np.float32)
    O2, lse2 = chunk_attention_ref(q, k + u, v, T, ln, w.prior, w.chunk, w.scale)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-5)
    shift = w.scale * (q.astype(np.float64) @ u.astype(np.float64))
    for b in range(w.B):
        C = w.chunk[b]
        np.testing.assert_allclose(lse2[b, :, :C], lse[b, :, :C] + shift[b, :, :C], atol=1e-4)


def test_poison_invariance_unselected_blocks_and_tail():
    w = _tiny(seed=13, prior=(256, 320), chunk=(128, 64), p=0.25, L=512)
    q, k, v = _arrays(w)
    T, ln = _tables(w)
    O, lse = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    kp, vp = k.copy(), v.copy()
    for b in range(w.B):
        for g in range(w.H_kv):
            sel = set(T[b, g, :ln[b, g]].tolist())
            for kb in range(w.L // 64):
                if kb not in sel:
                    kp[b, g, kb * 64:(kb + 1) * 64] = np.nan
                    vp[b, g, kb * 64:(kb + 1) * 64] = np.nan
            kp[b, g, w.prior[b] + w.chunk[b]:] = np.nan
            vp[b, g, w.prior[b] + w.chunk[b]:] = np.nan
    O2, lse2 = chunk_attention_ref(q, kp, vp, T, ln, w.prior, w.chunk, w.scale)
    np.testing.assert_array_equal(O2, O)
    np.testing.assert_array_equal(lse2, lse)
    assert np.all(np.isfinite(O2))


def test_sparse_selection_changes_result():
    # The union table matters: dropping a selected block changes the rows that saw it.
    w = _tiny(seed=14, p=0.3)
    q, k, v = _arrays(w)
    T, ln = _tables(w)
    O, _ = chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)
    T2, ln2 = T.copy(), ln.copy()
    T2[0, 0, :ln[0, 0] - 1] = T[0, 0, 1:ln[0, 0]]
    T2[0, 0, ln[0, 0] - 1] = -1
    ln2[0, 0] -= 1
    O2, _ = chunk_attention_ref(q, k, v, T2, ln2, w.prior, w.chunk, w.scale)
    assert np.abs(O2[0, :w.G] - O[0, :w.G]).max() > 1e-3
    np.testing.assert_array_equal(O2[1], O[1])
