"""GPU parity of the block-sparse-execution baseline (through the C ABI).

Each 64-row Q-block of each head attends its own mask row (no union): the
per-row lists come from ca_build_union_tables on the mask viewed as one-row
groups, and ca_chunk_attention_rows runs them.  Compared with the float64
oracle ``sparse_attention_ref``: lists bit-exact, outputs within the same
bounds as the union attention.
"""
import zlib

import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from oracle import sparse_attention_ref, sparse_attention_rows_ref
from tests.gpu_util import (F32_MAX_ABS, check_lse, Dev, compare_bf16, f32_arrays, sample_rows, say,
                            to_np)

pytestmark = pytest.mark.gpu


def _bern(p):
    return lambda rng, b, H, nq, pb: (rng.random((H, nq, pb)) < p).astype(np.uint8)


def _run(w):
    d = Dev(w)
    T, lens = ca.build_row_tables(d.mask, w.n_kv_blocks)
    O, lse = ca.chunk_attention_rows(d.q, d.k, d.v, T, lens, w.prior, w.chunk, w.scale,
                                     return_lse=True)
    torch.cuda.synchronize()
    return d, T, lens, O, lse


def _check_lists(w, T, lens):
    T = T.cpu().numpy()
    lens = lens.cpu().numpy()
    for b in range(w.B):
        nkb = w.n_kv_blocks[b]
        for h in range(w.H_q):
            for qb in range(w.mask.shape[2]):
                sel = np.flatnonzero(w.mask[b, h, qb, :nkb])
                assert lens[b, h, qb] == sel.size
                assert T[b, h, qb, :sel.size].tolist() == sel.tolist()
                assert (T[b, h, qb, sel.size:] == -1).all()


SMALL = [
    # dtype, B, H_q, H_kv, D, prior, chunk, C_max
    ("bf16", 1, 8, 2, 128, [2048], [256], 256),
    ("bf16", 3, 8, 1, 64, [1024, 0, 3072], [192, 128, 320], 384),
    ("bf16", 2, 4, 4, 128, [512, 1536], [64, 0], 128),
    ("f32", 2, 4, 2, 128, [640, 192], [192, 128], 256),
    ("f32", 1, 8, 1, 64, [1024], [256], 320),
]


@pytest.mark.parametrize("dtype,B,H_q,H_kv,D,prior,chunk,C_max", SMALL)
def test_sparse_small_full_parity(dtype, B, H_q, H_kv, D, prior, chunk, C_max):
    w = gen.make_custom(B, H_q, H_kv, D, prior, chunk, dtype, 4242 + D + B, _bern(0.2),
                        C_max=C_max, name=f"sparse_small_{dtype}")
    say(f"sparse small {dtype} B={B} H={H_q}/{H_kv} D={D} prior={prior} chunk={chunk}")
    d, T, lens, O, lse = _run(w)
    _check_lists(w, T, lens)
    q, k, v = f32_arrays(w)
    Or, lr = sparse_attention_ref(q, k, v, w.mask, w.prior, w.chunk, w.scale)
    got, gl = to_np(O), lse.cpu().numpy()
    if dtype == "f32":
        np.testing.assert_allclose(got, Or, rtol=0, atol=F32_MAX_ABS)
        check_lse(gl, lr, fp32=True)
    else:
        compare_bf16(got, Or, "O")
        fin = np.isfinite(lr)
        assert (np.isfinite(gl) == fin).all()
        check_lse(gl[fin], lr[fin])


@pytest.mark.parametrize("variant", ["pairwise", "colshared", "groupshared"])
def test_sparse_full_size_128k_sampled(variant):
    say(f"sparse llama8b_128k {variant}")
    w = gen.make_workload("llama8b_128k", variant=variant)
    d, T, lens, O, lse = _run(w)
    say(f"  mean per-row list {float(lens.float().mean()):.1f} blocks")
    rows = sample_rows(w, seed=zlib.crc32(variant.encode()) % 1000)
    q, k, v = f32_arrays(w)
    Or, lr = sparse_attention_rows_ref(q, k, v, w.mask, w.prior, w.chunk, w.scale, rows)
    r = torch.from_numpy(rows).cuda()
    compare_bf16(to_np(O[r[:, 0], r[:, 1], r[:, 2]]), Or, f"{len(rows)} sampled rows")
    check_lse(to_np(lse[r[:, 0], r[:, 1], r[:, 2]]), lr)
    assert bool(torch.isfinite(O).all())
    # per-row lists against the mask on a few rows (the whole check is slow in Python)
    Th, lh = T.cpu().numpy(), lens.cpu().numpy()
    for h, qb in ((0, 0), (5, 17), (31, 31)):
        sel = np.flatnonzero(w.mask[0, h, qb, :w.n_kv_blocks[0]])
        assert lh[0, h, qb] == sel.size and Th[0, h, qb, :sel.size].tolist() == sel.tolist()


def test_sparse_poison_invariance():
    # NaN in every cache row that no list of its KV head selects leaves O unchanged
    w = gen.make_custom(2, 8, 2, 128, [4096, 2048], [256, 192], "bf16", 99, _bern(0.1),
                        C_max=256, name="sparse_poison")
    say("sparse poison invariance")
    d, T, lens, O, _ = _run(w)
    keep = np.zeros((w.B, w.H_kv, w.L), bool)
    for b in range(w.B):
        for h in range(w.H_q):
            for qb in range(-(-w.chunk[b] // 64)):
                for kb in np.flatnonzero(w.mask[b, h, qb, :w.n_kv_blocks[b]]):
                    keep[b, h // w.G, kb * 64:(kb + 1) * 64] = True
        keep[b, :, w.prior[b] + w.chunk[b]:] = False
    kp, vp = d.k.clone(), d.v.clone()
    km = torch.from_numpy(~keep).cuda()
    kp[km] = float("nan")
    vp[km] = float("nan")
    O2 = ca.chunk_attention_rows(d.q, kp, vp, T, lens, w.prior, w.chunk, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
