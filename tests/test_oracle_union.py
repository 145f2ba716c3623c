"""Pins for the Block-Union oracle (CPU only).

The pages give the union only as a definition (coverage-preserving, minimal,
built by a Q-block union and an intra-group union; CompactAttention
"Methodology" and abstract) and print no worked example.  The oracle is pinned
here by a hand-worked fixture, brute force with Python sets, set invariants,
special cases and a closed-form statistic of the synthetic masks.
"""
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import gen
from oracle import check_tables_ref, tables_to_csr_ref, union_tables_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "union_hand_worked.txt")


def _read_golden():
    mask = np.zeros((1, 4, 3, 6), np.uint8)
    tables, ln, indptr, indices = {}, None, None, None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, vals = line.partition(":")
        head = key.split()
        nums = [int(x) for x in vals.split()]
        if head[0] == "mask":
            mask[0, int(head[1]), int(head[2])] = nums
        elif head[0] == "table":
            tables[int(head[1])] = nums
        elif head[0] == "len":
            ln = nums
        elif head[0] == "indptr":
            indptr = nums
        elif head[0] == "indices":
            indices = nums
    return mask, tables, ln, indptr, indices


def brute_force_union(mask, H_kv, nq, nkb):
    """Python-set brute force of the definition, one cell at a time."""
    B, H_q, _, NKB_max = mask.shape
    G = H_q // H_kv
    T = np.full((B, H_kv, NKB_max), -1, np.int32)
    ln = np.zeros((B, H_kv), np.int32)
    for b in range(B):
        for g in range(H_kv):
            chosen = set()
            for h in range(g * G, g * G + G):
                for qb in range(nq[b]):
                    for kb in range(nkb[b]):
                        if mask[b, h, qb, kb]:
                            chosen.add(kb)
            lst = sorted(chosen)
            T[b, g, :len(lst)] = lst
            ln[b, g] = len(lst)
    return T, ln


def _random_case(rng):
    H_kv = int(rng.integers(1, 4))
    G = int(rng.integers(1, 5))
    B = int(rng.integers(1, 4))
    NQ_max = int(rng.integers(1, 5))
    NKB_max = int(rng.integers(1, 40))
    nq = [int(rng.integers(0, NQ_max + 1)) for _ in range(B)]
    nkb = [int(rng.integers(0, NKB_max + 1)) for _ in range(B)]
    p = float(rng.uniform(0.0, 0.5))
    mask = (rng.random((B, H_kv * G, NQ_max, NKB_max)) < p).astype(np.uint8)
    return mask, H_kv, nq, nkb


def test_hand_worked_fixture():
    mask, tables, ln, indptr, indices = _read_golden()
    T, L_ = union_tables_ref(mask, 2, [2], [5])
    assert T[0, 0].tolist() == tables[0]
    assert T[0, 1].tolist() == tables[1]
    assert L_[0].tolist() == ln
    ip, ix = tables_to_csr_ref(T, L_, L=384)
    assert ip.tolist() == indptr
    assert ix.tolist() == indices


def test_brute_force_seeded():
    rng = np.random.default_rng(7)
    for _ in range(300):
        mask, H_kv, nq, nkb = _random_case(rng)
        T, ln = union_tables_ref(mask, H_kv, nq, nkb)
        Tb, lnb = brute_force_union(mask, H_kv, nq, nkb)
        np.testing.assert_array_equal(T, Tb)
        np.testing.assert_array_equal(ln, lnb)


@settings(max_examples=150, deadline=None)
@given(st.integers(0, 2**31 - 1))
def test_brute_force_hypothesis(seed):
    rng = np.random.default_rng(seed)
    mask, H_kv, nq, nkb = _random_case(rng)
    # nonzero bytes other than 1 count as selected too
    mask = mask * rng.integers(1, 256, size=mask.shape).astype(np.uint8)
    T, ln = union_tables_ref(mask, H_kv, nq, nkb)
    Tb, lnb = brute_force_union(mask, H_kv, nq, nkb)
    np.testing.assert_array_equal(T, Tb)
    np.testing.assert_array_equal(ln, lnb)


def test_invariants_coverage_minimality_order():
    rng = np.random.default_rng(11)
    for _ in range(100):
        mask, H_kv, nq, nkb = _random_case(rng)
        T, ln = union_tables_ref(mask, H_kv, nq, nkb)
        B, H_q, _, NKB_max = mask.shape
        G = H_q // H_kv
        for b in range(B):
            for g in range(H_kv):
                row = T[b, g]
                n = int(ln[b, g])
                sel = row[:n]
                assert np.all(row[n:] == -1)
                assert np.all(np.diff(sel) > 0)  # strictly ascending
                assert np.all((sel >= 0) & (sel < nkb[b]))
                cells = mask[b, g * G:(g + 1) * G, :nq[b], :nkb[b]]
                # coverage: every selected cell's block is in T
                for kb in np.argwhere(cells)[:, 2]:
                    assert kb in set(sel.tolist())
                # minimality: each block in T was selected by some head / Q-block
                for kb in sel:
                    assert cells[:, :, kb].any()


def test_homomorphism_and_monotonicity():
    rng = np.random.default_rng(3)
    for _ in range(60):
        m1, H_kv, nq, nkb = _random_case(rng)
        m2 = (rng.random(m1.shape) < 0.2).astype(np.uint8)
        T1, l1 = union_tables_ref(m1, H_kv, nq, nkb)
        T2, l2 = union_tables_ref(m2, H_kv, nq, nkb)
        T12, l12 = union_tables_ref(m1 | m2, H_kv, nq, nkb)
        for b in range(m1.shape[0]):
            for g in range(H_kv):
                s1 = set(T1[b, g, :l1[b, g]].tolist())
                s2 = set(T2[b, g, :l2[b, g]].tolist())
                s12 = set(T12[b, g, :l12[b, g]].tolist())
                assert s12 == s1 | s2
                assert s1 <= s12 and s2 <= s12


def test_special_cases():
    B, H_q, H_kv, NQ, NKB = 2, 8, 2, 3, 17
    nq, nkb = [3, 2], [17, 9]
    ones = np.ones((B, H_q, NQ, NKB), np.uint8)
    T, ln = union_tables_ref(ones, H_kv, nq, nkb)
    for b in range(B):
        for g in range(H_kv):
            assert T[b, g, :ln[b, g]].tolist() == list(range(nkb[b]))
            assert np.all(T[b, g, ln[b, g]:] == -1)
    zeros = np.zeros_like(ones)
    T, ln = union_tables_ref(zeros, H_kv, nq, nkb)
    assert np.all(ln == 0) and np.all(T == -1)
    one = zeros.copy()
    one[1, 5, 1, 4] = 1  # head 5 -> group 1 (G = 4)
    T, ln = union_tables_ref(one, H_kv, nq, nkb)
    assert ln.tolist() == [[0, 0], [0, 1]]
    assert T[1, 1, 0] == 4


def test_cells_outside_extent_ignored():
    rng = np.random.default_rng(5)
    for _ in range(50):
        mask, H_kv, nq, nkb = _random_case(rng)
        T, ln = union_tables_ref(mask, H_kv, nq, nkb)
        poisoned = mask.copy()
        for b in range(mask.shape[0]):
            poisoned[b, :, nq[b]:, :] = 1
            poisoned[b, :, :, nkb[b]:] = 1
        T2, ln2 = union_tables_ref(poisoned, H_kv, nq, nkb)
        np.testing.assert_array_equal(T, T2)
        np.testing.assert_array_equal(ln, ln2)


def test_group_mapping_consecutive_heads():
    # Query head h belongs to group h // G: selecting in head G (first head of group 1)
    # must land in group 1, never in group 0 (a mapping h % H_kv would put it in group 0).
    H_q, H_kv = 8, 2
    mask = np.zeros((1, H_q, 1, 8), np.uint8)
    mask[0, 1, 0, 3] = 1  # head 1 -> group 0
    mask[0, 4, 0, 6] = 1  # head 4 -> group 1
    T, ln = union_tables_ref(mask, H_kv, [1], [8])
    assert T[0, 0, :ln[0, 0]].tolist() == [3]
    assert T[0, 1, :ln[0, 1]].tolist() == [6]


def test_csr_view_roundtrip():
    rng = np.random.default_rng(9)
    for _ in range(30):
        mask, H_kv, nq, nkb = _random_case(rng)
        T, ln = union_tables_ref(mask, H_kv, nq, nkb)
        pages = -(-mask.shape[3] // 1)
        L = pages * 64
        ip, ix = tables_to_csr_ref(T, ln, L)
        B = mask.shape[0]
        assert ip[0] == 0 and ip[-1] == ln.sum() and np.all(np.diff(ip) == ln.reshape(-1))
        for u in range(B * H_kv):
            b, g = divmod(u, H_kv)
            seg = ix[ip[u]:ip[u + 1]]
            assert np.all(seg // pages == u)
            assert (seg % pages).tolist() == T[b, g, :ln[b, g]].tolist()


def _union_fraction(w, forced):
    """Mean fraction of non-forced prior blocks present in T, over all groups."""
    T, ln = union_tables_ref(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
    hits, trials = 0, 0
    for b in range(w.B):
        p_blk = w.prior[b] // 64
        free = [kb for kb in range(p_blk) if kb not in forced(p_blk)]
        fs = set(free)
        for g in range(w.H_kv):
            s = set(T[b, g, :ln[b, g]].tolist())
            hits += len(s & fs)
            trials += len(free)
    return hits, trials


@pytest.mark.parametrize("variant,expo", [("colshared", "G"), ("pairwise", "G*NQ"),
                                          ("groupshared", "1")])
def test_statistic_union_density_128k(variant, expo):
    w = gen.make_workload("llama8b_128k", variant=variant, with_tensors=False)
    hits, n = _union_fraction(w, lambda p_blk: {0} | set(range(p_blk - 8, p_blk)))
    e = {"G": w.G, "G*NQ": w.G * 32, "1": 1}[expo]
    p = 1 - (1 - 0.05) ** e  # closed form: block missed by all e independent cells
    sigma = math.sqrt(n * p * (1 - p))
    assert abs(hits - n * p) <= 5 * sigma + 1e-9, (hits, n * p, sigma)


def test_statistic_union_density_custom():
    # sparser pairwise mask so the closed form is far from 0 and 1
    pr = 0.02
    w = gen.make_custom(1, 8, 2, 64, [64 * 3000], [256], "bf16", 77,
                        lambda rng, b, H, nq, pb: (rng.random((H, nq, pb)) < pr).astype(np.uint8),
                        with_tensors=False)
    hits, n = _union_fraction(w, lambda p_blk: set())
    p = 1 - (1 - pr) ** (4 * 4)
    sigma = math.sqrt(n * p * (1 - p))
    assert abs(hits - n * p) <= 5 * sigma, (hits, n * p, sigma)


def test_generators_current_chunk_blocks_always_selected():
    for name in ("tiny_f32", "llama8b_32k", "ragged_b4"):
        w = gen.make_workload(name, with_tensors=False)
        T, ln = union_tables_ref(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
        for b in range(w.B):
            p_blk = w.prior[b] // 64
            for g in range(w.H_kv):
                s = set(T[b, g, :ln[b, g]].tolist())
                assert set(range(p_blk, w.n_kv_blocks[b])) <= s
                assert 0 in s  # sink


def test_table_contract_check():
    # Tables from the union pass; each planted violation raises exactly its own
    # flag (1 len out of range, 2 entry out of range, 4 not strictly
    # ascending, 8 padding other than -1).
    rng = np.random.default_rng(5)
    mask = (rng.random((2, 4, 3, 12)) < 0.3).astype(np.uint8)
    nkb = [12, 9]
    T, ln = union_tables_ref(mask, 2, [3, 2], nkb)
    assert not check_tables_ref(T, ln, nkb, 12).any()
    # a row with at least two entries and room for padding
    b, g = next((b, g) for b in range(2) for g in range(2) if 2 <= ln[b, g] < 12)
    n = int(ln[b, g])

    def planted(fn):
        T2, l2 = T.copy(), ln.copy()
        fn(T2, l2)
        return check_tables_ref(T2, l2, nkb, 12)

    cases = [
        (lambda T2, l2: l2.__setitem__((b, g), 13), 1 | 8 * 0),
        (lambda T2, l2: l2.__setitem__((b, g), -1), None),
        (lambda T2, l2: T2.__setitem__((b, g, 0), nkb[b]), None),
        (lambda T2, l2: T2.__setitem__((b, g, 1), T2[b, g, 0]), 4),
        (lambda T2, l2: T2.__setitem__((b, g, n), 0), 8),
    ]
    # len 13 > NKB_max: flag 1; the row is then judged over all 12 entries,
    # whose -1 padding breaks range and ascent too
    got = planted(cases[0][0])
    assert got[b, g] & 1 and got[b, g] & 2
    # negative len: flag 1, and the real entries now count as bad padding
    got = planted(cases[1][0])
    assert got[b, g] == 1 | 8
    # entry past the sequence's blocks: flag 2 (and ascent, if it exceeds the next)
    got = planted(cases[2][0])
    assert got[b, g] & 2
    assert planted(cases[3][0])[b, g] == 4
    assert planted(cases[4][0])[b, g] == 8
    for c in cases:  # the other rows are untouched
        got = planted(c[0])
        others = np.ones((2, 2), bool)
        others[b, g] = False
        assert not got[others].any()

