"""GPU parity of the block-mask producer (through the C ABI).

Pooling and scores are floating point: compared with the float64 oracle
within their rounding bounds (the scores: products of bf16 hi/lo parts of the
fp32 pooled values, within 2^-14 of sum_d |q_d k_d|, tests/gpu_util.py).  The
selection turns scores into bits, so it is checked bit-exact against the
oracle's selection fed the GPU's own fp32 scores (both sides decide in the
kernel's precision); the whole producer is then compared with the float64
oracle end to end, where rows may differ only if the oracle's scores at the
budget boundary are within the score bound.
"""
import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from oracle import block_scores_ref, pool_blocks_ref, producer_mask_ref, topk_mask_ref
from tests.gpu_util import check_scores, say, score_bound

pytestmark = pytest.mark.gpu

POOL_ATOL = 2e-6    # |mean of 64 values| error in fp32: a few ulps of the partial sums


def _f32(t):
    return gen.tensor_to_f32(t.detach().cpu())


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_pool_blocks(dtype, D):
    rng = np.random.default_rng(D)
    B, H, R = 3, 4, 40 * 64
    x32 = rng.standard_normal((B, H, R, D)).astype(np.float32)
    x = torch.from_numpy(x32)
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    xr = gen.tensor_to_f32(x)
    lo, hi = [0, 5, 39], [40, 17, 39]
    out = torch.full((B, H, 41, D), 7.0, device="cuda")
    ca.pool_blocks(x.cuda(), lo, hi, out=out)
    torch.cuda.synchronize()
    ref = pool_blocks_ref(xr, lo, hi, 41)
    got = out.cpu().numpy()
    have = ~np.isnan(ref)
    np.testing.assert_allclose(got[have], ref[have], rtol=0, atol=POOL_ATOL)
    assert (got[~have] == 7.0).all()  # untouched outside the ranges


def _producer(w, budget, local):
    d_q = w.q.cuda()
    d_k = w.k.cuda()
    NQ_max = -(-w.C_max // 64)
    qbar = ca.pool_blocks(d_q, [0] * w.B, [c // 64 for c in w.chunk], n_out=NQ_max)
    kbar = ca.pool_blocks(d_k, [0] * w.B, [p // 64 for p in w.prior], n_out=w.NKB_max)
    mask, scores = ca.block_mask_topk(qbar, kbar, w.prior, w.chunk, budget, local)
    torch.cuda.synchronize()
    return qbar, kbar, mask, scores


def _check(w, budget, local):
    qbar, kbar, mask, scores = _producer(w, budget, local)
    q, k = gen.tensor_to_f32(w.q), gen.tensor_to_f32(w.k)
    NQ_max = qbar.shape[2]
    qr = np.nan_to_num(pool_blocks_ref(q, [0] * w.B, [c // 64 for c in w.chunk], NQ_max))
    kr = np.nan_to_num(pool_blocks_ref(k, [0] * w.B, [p // 64 for p in w.prior], w.NKB_max))
    sr = block_scores_ref(qr, kr)
    tol = score_bound(qr, kr)
    sg = scores.cpu().numpy().astype(np.float64)
    m = mask.cpu().numpy()
    for b in range(w.B):
        nq, P = w.chunk[b] // 64, w.prior[b] // 64
        check_scores(sg[b, :, :nq, :P], sr[b, :, :nq, :P], tol[b, :, :nq, :P], f"scores b={b}")
    # selection: bit-exact on the GPU's own scores
    sel_in = np.zeros_like(sg)
    for b in range(w.B):
        nq, P = w.chunk[b] // 64, w.prior[b] // 64
        sel_in[b, :, :nq, :P] = sg[b, :, :nq, :P]
    ref_bits = topk_mask_ref(sel_in, w.prior, w.chunk, budget, local, w.NKB_max)
    np.testing.assert_array_equal(m, ref_bits)
    # end to end against the float64 producer: differing rows must be ambiguous
    full = producer_mask_ref(q, k, w.prior, w.chunk, budget, local, w.NKB_max)
    bad = np.argwhere((full != m).any(axis=3))
    for b, h, qb in bad:
        P = w.prior[b] // 64
        lo = max(P - local, 1)
        s = np.sort(sr[b, h, qb, 1:lo])[::-1]
        gap = s[budget - 1] - s[budget] if budget < s.size else np.inf
        assert gap <= 2 * tol[b, h, qb, 1:lo].max(), (b, h, qb, gap)
    say(f"  rows {m.shape[0] * m.shape[1] * m.shape[2]}, ambiguous-row differences {len(bad)}")
    return m


@pytest.mark.parametrize("budget,local", [(0, 4), (3, 0), (8, 2), (500, 4)])
def test_producer_small(budget, local):
    w = gen.make_custom(3, 8, 2, 128, [64 * 60, 0, 64 * 7], [256, 128, 192], "bf16", 31,
                        lambda rng, b, H, nq, pb: np.zeros((H, nq, pb), np.uint8), C_max=320,
                        name="producer_small")
    say(f"producer small budget={budget} local={local}")
    _check(w, budget, local)


def test_producer_ties_lower_block_first():
    # K blocks repeated so that many block scores tie exactly
    w = gen.make_custom(1, 4, 1, 64, [64 * 48], [128], "f32", 5,
                        lambda rng, b, H, nq, pb: np.zeros((H, nq, pb), np.uint8),
                        name="producer_ties")
    k = w.k.clone()
    base = k[:, :, 64:128].clone()
    for kb in range(1, 48):
        k[:, :, kb * 64:(kb + 1) * 64] = base if kb % 3 else base * 0.5
    w.k = k
    say("producer ties")
    m = _check(w, budget=5, local=2)
    row = np.flatnonzero(m[0, 0, 0, 1:46]) + 1
    assert row.tolist() == [1, 2, 4, 5, 7]  # equal scores: lowest kb first


def test_producer_full_size_128k():
    w = gen.make_workload("llama8b_128k", variant="pairwise")
    say("producer llama8b_128k budget=64 local=8")
    m = _check(w, budget=64, local=8)
    assert (m[0, :, :, 1:2016 - 8].sum(axis=2) >= 0).all()
    assert (m[0, :, :, 1:2016 - 8].sum(axis=-1) == 64).all()


@pytest.mark.parametrize("NKB", [15360, 16064])
def test_topk_long_rows(NKB):
    # the top-k stages a row's keys in LDS up to 15360 blocks and reads them
    # from the scores in global memory past that: both sides of the limit, with
    # exact ties (repeated pooled keys) among thousands of candidates
    rng = np.random.default_rng(NKB)
    B, H_q, H_kv, D, C = 1, 2, 1, 64, 128
    P = (NKB - C // 64) * 64
    pblk = P // 64
    qbar = rng.standard_normal((B, H_q, C // 64, D)).astype(np.float32)
    kbar = rng.standard_normal((B, H_kv, NKB, D)).astype(np.float32)
    kbar[:, :, 1::7] = kbar[:, :, 1:2]
    d_q, d_k = torch.from_numpy(qbar).cuda(), torch.from_numpy(kbar).cuda()
    for budget, local in ((64, 8), (3000, 0), (1, 3)):
        say(f"top-k long rows NKB={NKB} budget={budget} local={local}")
        mask, scores = ca.block_mask_topk(d_q, d_k, [P], [C], budget, local)
        torch.cuda.synchronize()
        sel_in = np.zeros((B, H_q, C // 64, pblk), np.float64)
        sel_in[...] = scores.cpu().numpy()[:, :, :, :pblk]
        ref = topk_mask_ref(sel_in, [P], [C], budget, local, NKB)
        np.testing.assert_array_equal(mask.cpu().numpy(), ref)


@pytest.mark.parametrize("seed", range(16))
def test_producer_fuzz(seed):
    # seeded random batch, heads, group size, head dim, element type, ragged
    # prior / chunk lengths (zero included), padding, budget and local window
    rng = np.random.default_rng(30_000 + seed)
    H_kv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 5))
    D = int(rng.choice([64, 128]))
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    prior = [64 * int(rng.integers(0, 80)) for _ in range(B)]
    chunk = [64 * int(rng.integers(0, 6)) for _ in range(B)]
    if max(chunk) == 0:
        chunk[0] = 64
    C_max = max(chunk) + 64 * int(rng.integers(0, 2))
    budget = int(rng.choice([0, 1, 5, 16, 100]))
    local = int(rng.choice([0, 1, 3, 8]))
    w = gen.make_custom(B, G * H_kv, H_kv, D, prior, chunk, dtype, 40_000 + seed,
                        lambda r, b, H, nq, pb: np.zeros((H, nq, pb), np.uint8), C_max=C_max,
                        name=f"producer_fuzz{seed}")
    say(f"producer fuzz {seed}: B={B} H={G * H_kv}/{H_kv} D={D} {dtype} prior={prior} "
        f"chunk={chunk} C_max={C_max} budget={budget} local={local}")
    _check(w, budget, local)
