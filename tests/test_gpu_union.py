"""GPU parity of the Block-Union table builder (through the C ABI): bit-exact
against the oracle, padding included, on every named workload, fuzzed tiny
shapes, ragged extents and both load paths (16-byte rows and byte rows)."""
import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from oracle import check_tables_ref, tables_to_csr_ref, union_tables_ref
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _gpu_tables(mask, H_kv, nq, nkb, garbage=True):
    m = torch.from_numpy(np.ascontiguousarray(mask)).cuda()
    B, _, _, NKB = mask.shape
    T = torch.full((B, H_kv, NKB), 12345, dtype=torch.int32, device="cuda") if garbage else None
    lens = torch.full((B, H_kv), -7, dtype=torch.int32, device="cuda") if garbage else None
    T, lens = ca.build_union_tables(m, H_kv, nq, nkb, T=T, lens=lens)
    torch.cuda.synchronize()
    return T.cpu().numpy(), lens.cpu().numpy()


def _check(mask, H_kv, nq, nkb, what=""):
    T, ln = _gpu_tables(mask, H_kv, nq, nkb)
    Tr, lr = union_tables_ref(mask, H_kv, nq, nkb)
    np.testing.assert_array_equal(ln, lr, err_msg=f"len {what}")
    np.testing.assert_array_equal(T, Tr, err_msg=f"T {what}")
    return T, ln


def test_union_fuzz_tiny():
    rng = np.random.default_rng(2024)
    say("union fuzz: 300 tiny cases")
    for case in range(300):
        H_kv = int(rng.integers(1, 5))
        G = int(rng.integers(1, 9))
        B = int(rng.integers(1, 5))
        NQ = int(rng.integers(1, 6))
        NKB = int(rng.choice([int(rng.integers(1, 80)), 16 * int(rng.integers(1, 9))]))
        nq = [int(rng.integers(0, NQ + 1)) for _ in range(B)]
        nkb = [int(rng.integers(0, NKB + 1)) for _ in range(B)]
        p = float(rng.uniform(0, 0.6))
        mask = (rng.random((B, H_kv * G, NQ, NKB)) < p).astype(np.uint8)
        mask *= rng.integers(1, 256, size=mask.shape).astype(np.uint8)
        _check(mask, H_kv, nq, nkb, what=f"case {case}")


@pytest.mark.parametrize("name,kw", [
    ("tiny_f32", {}),
    ("llama8b_32k", {}),
    ("llama8b_128k", dict(variant="pairwise")),
    ("llama8b_128k", dict(variant="colshared")),
    ("llama8b_128k", dict(variant="dense")),
    ("llama8b_128k", dict(variant="groupshared")),
    ("ragged_b4", {}),
] + [("vslash_128k", dict(density=d, heads=m)) for d in gen.VSLASH_DENSITIES
     for m in ("identical", "independent")])
def test_union_named_workloads(name, kw):
    w = gen.make_workload(name, with_tensors=False, **kw)
    say(f"union {name} {kw}: mask {w.mask.shape}")
    T, ln = _check(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks, what=name)
    say(f"  sum len {int(ln.sum())}, mean len {float(ln.mean()):.1f}")


def test_union_ignores_cells_outside_extent():
    w = gen.make_workload("ragged_b4", with_tensors=False)
    mask = w.mask.copy()
    for b in range(w.B):
        mask[b, :, w.n_q_blocks[b]:, :] = 1
        mask[b, :, :, w.n_kv_blocks[b]:] = 1
    T, ln = _gpu_tables(mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
    Tr, lr = union_tables_ref(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
    np.testing.assert_array_equal(T, Tr)
    np.testing.assert_array_equal(ln, lr)


@pytest.mark.parametrize("NKB,vec", [(40000, "byte rows"), (40960, "16-byte rows")])
def test_union_long_tables(NKB, vec):
    # more bitmap words than threads: each thread compacts several words
    rng = np.random.default_rng(NKB)
    mask = (rng.random((2, 4, 2, NKB)) < 0.3).astype(np.uint8)
    say(f"union long tables NKB={NKB} ({vec})")
    _check(mask, 2, [2, 1], [NKB, NKB - 77], what=vec)


def test_union_single_cell_and_empty():
    mask = np.zeros((1, 8, 4, 64), np.uint8)
    T, ln = _check(mask, 2, [4], [64])
    assert np.all(ln == 0) and np.all(T == -1)
    mask[0, 6, 3, 63] = 1
    T, ln = _check(mask, 2, [4], [64])
    assert ln.tolist() == [[0, 1]] and T[0, 1, 0] == 63


def test_csr_view_matches_oracle():
    w = gen.make_workload("ragged_b4", with_tensors=False)
    m = torch.from_numpy(w.mask).cuda()
    T, lens = ca.build_union_tables(m, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
    indptr, indices = ca.tables_to_csr(T, lens, w.L)
    torch.cuda.synchronize()
    Tr, lr = union_tables_ref(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
    ip_r, ix_r = tables_to_csr_ref(Tr, lr, w.L)
    ip = indptr.cpu().numpy()
    np.testing.assert_array_equal(ip, ip_r)
    np.testing.assert_array_equal(indices.cpu().numpy()[:ip[-1]], ix_r)


def test_check_tables_parity():
    # The contract check: every union table passes; fuzzed tables (entries
    # and lengths drawn around the valid ranges, some rows sorted, some padded
    # correctly) give the oracle's flags bit for bit.
    rng = np.random.default_rng(77)
    mask = (rng.random((3, 8, 4, 200)) < 0.05).astype(np.uint8)
    nq, nkb = [4, 2, 3], [200, 130, 77]
    T, ln = _gpu_tables(mask, 2, nq, nkb)
    Td, ld = torch.from_numpy(T).cuda(), torch.from_numpy(ln).cuda()
    bad = ca.check_tables(Td, ld, nkb)
    torch.cuda.synchronize()
    assert not bad.any(), bad
    for trial in range(20):
        B, H_kv, NKB = 3, 4, int(rng.integers(1, 300))
        nk = [int(rng.integers(0, NKB + 1)) for _ in range(B)]
        Tf = rng.integers(-2, NKB + 3, size=(B, H_kv, NKB)).astype(np.int32)
        lf = rng.integers(-1, NKB + 2, size=(B, H_kv)).astype(np.int32)
        for b in range(B):
            for g in range(H_kv):
                r = rng.random()
                if r < 0.5:  # a well-formed row, maybe one entry disturbed
                    n = int(rng.integers(0, nk[b] + 1))
                    row = np.sort(rng.choice(nk[b], size=n, replace=False)) if n else []
                    Tf[b, g] = -1
                    Tf[b, g, :n] = row
                    lf[b, g] = n
                    if r < 0.25 and NKB > 1:
                        Tf[b, g, int(rng.integers(0, NKB))] = int(rng.integers(-2, NKB + 3))
        want = check_tables_ref(Tf, lf, nk, NKB)
        got = ca.check_tables(torch.from_numpy(Tf).cuda(), torch.from_numpy(lf).cuda(), nk)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=f"trial {trial}")

