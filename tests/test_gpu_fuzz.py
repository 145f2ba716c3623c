"""Seeded random shapes through every attention entry point (whole tables,
split, balanced, per-Q-block lists), against the float64 oracle: batch, head
counts and group size, head dim, ragged prior and chunk lengths (zero
included), C_max padding, element type and mask density all drawn at random.  Tables are compared bit-exact, outputs at the stated
bounds (bf16: max-abs 2e-2, mean-abs 2e-3; fp32: max-abs 1e-5).
"""
import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from oracle import sparse_attention_ref
from tests.gpu_util import (F32_MAX_ABS, check_bf16_rounding, check_lse, Dev, compare_bf16,
                            oracle_full, oracle_full_absv, oracle_tables,
                            say, to_np)

pytestmark = pytest.mark.gpu

N_CASES = 120


def _case(seed):
    rng = np.random.default_rng(10_000 + seed)
    H_kv = int(rng.choice([1, 2, 3, 4]))
    G = int(rng.choice([1, 2, 3, 4, 8]))
    B = int(rng.integers(1, 5))
    D = int(rng.choice([64, 128]))
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    prior = [64 * int(rng.integers(0, 40)) for _ in range(B)]
    chunk = [64 * int(rng.integers(0, 6)) for _ in range(B)]
    if max(chunk) == 0:
        chunk[0] = 64
    C_max = max(chunk) + 64 * int(rng.integers(0, 2)) + int(rng.integers(0, 2)) * 17
    p = float(rng.choice([0.0, 0.05, 0.3, 1.0]))
    n_split = int(rng.choice([2, 3, 5, 16]))
    cell = lambda r, b, H, nq, pb: (r.random((H, nq, pb)) < p).astype(np.uint8)
    w = gen.make_custom(B, G * H_kv, H_kv, D, prior, chunk, dtype, 20_000 + seed, cell,
                        C_max=C_max, name=f"fuzz{seed}")
    return w, n_split


def _compare(w, O, lse, Or, lr, what, absv=None):
    if w.dtype == "bf16":
        compare_bf16(to_np(O), Or, what)
        if absv is not None:
            check_bf16_rounding(to_np(O), Or, absv, lr, what)
    else:
        err = float(np.abs(to_np(O) - Or).max())
        assert err <= F32_MAX_ABS, (what, err)
    check_lse(to_np(lse), lr, what, fp32=w.dtype != "bf16")
    for b in range(w.B):
        assert np.all(to_np(O)[b, :, w.chunk[b]:] == 0), what


@pytest.mark.parametrize("seed", range(N_CASES))
def test_fuzz_shapes_all_entry_points(seed):
    w, n_split = _case(seed)
    say(f"fuzz {seed}: B={w.B} H={w.H_q}/{w.H_kv} D={w.D} {w.dtype} prior={w.prior} "
        f"chunk={w.chunk} C_max={w.C_max} n_split={n_split}")
    d = Dev(w)
    T, lens = d.tables()
    Tr, lr_ = oracle_tables(w)
    np.testing.assert_array_equal(T.cpu().numpy(), Tr)
    np.testing.assert_array_equal(lens.cpu().numpy(), lr_)
    assert not ca.check_tables(T, lens, w.n_kv_blocks).any()
    Or, lr = oracle_full(w)
    O, lse = d.attention(T, lens, return_lse=True)
    Os, lses = ca.chunk_attention(d.q, d.k, d.v, T, lens, w.prior, w.chunk, w.scale,
                                  return_lse=True, n_splits=n_split)
    torch.cuda.synchronize()
    Ob, lseb = ca.chunk_attention(d.q, d.k, d.v, T, lens, w.prior, w.chunk, w.scale,
                                  return_lse=True, balanced=True)
    torch.cuda.synchronize()
    absv = oracle_full_absv(w) if w.dtype == "bf16" else None
    _compare(w, O, lse, Or, lr, "union", absv)
    _compare(w, Os, lses, Or, lr, f"union, {n_split} splits", absv)
    _compare(w, Ob, lseb, Or, lr, "union, balanced", absv)
    # block-sparse execution of the same mask (per-(head, Q-block) lists)
    Trw, lrw = ca.build_row_tables(d.mask, w.n_kv_blocks)
    Orw, lserw = ca.chunk_attention_rows(d.q, d.k, d.v, Trw, lrw, w.prior, w.chunk, w.scale,
                                         return_lse=True)
    torch.cuda.synchronize()
    q, k, v = (gen.tensor_to_f32(x) for x in (w.q, w.k, w.v))
    Osr, lsr = sparse_attention_ref(q, k, v, w.mask, w.prior, w.chunk, w.scale)
    _compare(w, Orw, lserw, Osr, lsr, "per-Q-block lists")
