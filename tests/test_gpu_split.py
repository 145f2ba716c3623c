"""GPU parity of split-KV attention (ca_chunk_attention_split) against the
float64 oracle: each (b, g) table cut into several ranges run by separate
workgroups, then merged.  The result must match the oracle at the same bounds
as the unsplit kernel, whatever the number of ranges (including ranges with
no block at all), and read only the listed blocks.
"""
import zlib

import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from tests.gpu_util import (F32_MAX_ABS, check_lse, Dev, compare_bf16, f32_arrays, oracle_full,
                            oracle_rows, sample_rows, say, to_np)

pytestmark = pytest.mark.gpu


def _bern(p):
    return lambda rng, b, H, nq, pb: (rng.random((H, nq, pb)) < p).astype(np.uint8)


def _split(d, T, lens, n, return_lse=True):
    w = d.w
    return ca.chunk_attention(d.q, d.k, d.v, T, lens, w.prior, w.chunk, w.scale,
                              return_lse=return_lse, n_splits=n)


SMALL = [
    # B, H_q, H_kv, D, prior, chunk, C_max, n_splits
    (1, 4, 1, 128, [4096], [256], 256, 2),
    (1, 4, 1, 128, [4096], [256], 256, 16),        # more ranges than a 32-row tile's blocks
    (3, 8, 2, 64, [1024, 0, 3072], [192, 128, 320], 384, 3),
    (2, 8, 1, 128, [640, 2048], [64, 256], 320, 4),
    (1, 32, 8, 128, [8192], [512], 512, 5),
]


@pytest.mark.parametrize("B,H_q,H_kv,D,prior,chunk,C_max,n", SMALL)
def test_split_small_full_parity(B, H_q, H_kv, D, prior, chunk, C_max, n):
    w = gen.make_custom(B, H_q, H_kv, D, prior, chunk, "bf16", 900 + n + D, _bern(0.2),
                        C_max=C_max, name="split_small")
    say(f"split small B={B} H={H_q}/{H_kv} D={D} prior={prior} chunk={chunk} n={n}")
    d = Dev(w)
    T, lens = d.tables()
    O, lse = _split(d, T, lens, n)
    O1, l1 = d.attention(T, lens, return_lse=True)
    torch.cuda.synchronize()
    Or, lr = oracle_full(w)
    compare_bf16(to_np(O), Or, f"split n={n}")
    gl = lse.cpu().numpy()
    fin = np.isfinite(lr)
    assert (np.isfinite(gl) == fin).all()
    check_lse(gl[fin], lr[fin])
    # the same admissible keys as the unsplit kernel: only merge rounding differs
    assert float((O.float() - O1.float()).abs().max()) <= 2e-2
    for b in range(B):
        assert bool((O[b, :, chunk[b]:] == 0).all())


SMALL_F32 = [
    # B, H_q, H_kv, D, prior, chunk, C_max, n_splits
    (1, 4, 1, 64, [1024], [256], 256, 8),           # the tiny fp32 shape
    (1, 4, 1, 64, [1024], [256], 256, 16),          # ranges with no block
    (2, 4, 2, 128, [512, 1024], [192, 128], 200, 3),
    (3, 2, 1, 64, [0, 64, 4096], [128, 64, 256], 256, 2),
]


@pytest.mark.parametrize("B,H_q,H_kv,D,prior,chunk,C_max,n", SMALL_F32)
def test_split_f32_small_full_parity(B, H_q, H_kv, D, prior, chunk, C_max, n):
    w = gen.make_custom(B, H_q, H_kv, D, prior, chunk, "f32", 950 + n + D, _bern(0.3),
                        C_max=C_max, name="split_f32")
    say(f"split f32 B={B} H={H_q}/{H_kv} D={D} prior={prior} chunk={chunk} n={n}")
    d = Dev(w)
    T, lens = d.tables()
    O, lse = _split(d, T, lens, n)
    O1 = d.attention(T, lens)
    torch.cuda.synchronize()
    Or, lr = oracle_full(w)
    assert np.abs(to_np(O) - Or).max() <= F32_MAX_ABS
    fin = np.isfinite(lr)
    gl = lse.cpu().numpy()
    assert (np.isfinite(gl) == fin).all()
    check_lse(gl[fin], lr[fin], fp32=True)
    assert float((O - O1).abs().max()) <= F32_MAX_ABS
    for b in range(B):
        assert bool((O[b, :, chunk[b]:] == 0).all())


def _tp_shard(variant):
    """One GPU's share of the 128K LLaMA-8B chunk under tensor parallelism over
    KV heads: 4 query heads and their one KV head."""
    colshared = variant == "colshared"
    from gen.workloads import _bernoulli_sink_local
    return gen.make_custom(1, 4, 1, 128, [129024], [2048], "bf16", 1008,
                           lambda rng, b, H, nq, pb: _bernoulli_sink_local(
                               rng, H, nq, pb, 0.05, 8, colshared=colshared),
                           name=f"tp_shard_128k_{variant}")


@pytest.mark.parametrize("variant,n", [("pairwise", 4), ("colshared", 4), ("pairwise", 7)])
def test_split_tp_shard_128k_sampled(variant, n):
    say(f"split tp-shard 128K {variant} n={n}")
    w = _tp_shard(variant)
    d = Dev(w)
    T, lens = d.tables()
    O, lse = _split(d, T, lens, n)
    torch.cuda.synchronize()
    rows = sample_rows(w, seed=zlib.crc32(f"{variant}{n}".encode()) % 1000, heads_per_group=4,
                       extra=16)
    Or, lr = oracle_rows(w, rows)
    r = torch.from_numpy(rows).cuda()
    compare_bf16(to_np(O[r[:, 0], r[:, 1], r[:, 2]]), Or, f"{len(rows)} sampled rows")
    check_lse(to_np(lse[r[:, 0], r[:, 1], r[:, 2]]), lr)
    assert bool(torch.isfinite(O).all())


def test_split_poison_invariance():
    w = gen.make_custom(1, 8, 2, 128, [16384], [512], "bf16", 77, _bern(0.1), name="split_poison")
    say("split poison invariance")
    d = Dev(w)
    T, lens = d.tables()
    O = _split(d, T, lens, 4, return_lse=False)
    Th, lh = T.cpu().numpy(), lens.cpu().numpy()
    keep = np.zeros((w.B, w.H_kv, w.L), bool)
    for g in range(w.H_kv):
        for kb in Th[0, g, :lh[0, g]]:
            keep[0, g, kb * 64:(kb + 1) * 64] = True
    km = torch.from_numpy(~keep).cuda()
    kp, vp = d.k.clone(), d.v.clone()
    kp[km] = float("nan")
    vp[km] = float("nan")
    O2 = ca.chunk_attention(d.q, kp, vp, T, lens, w.prior, w.chunk, w.scale, n_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
