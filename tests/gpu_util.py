"""Helpers shared by the GPU parity tests: move a workload to the device, run
the HIP path through the C ABI, run the oracle on the same inputs, sample
output rows at full sizes."""
import sys

import numpy as np
import torch

import gen
import chunked_prefill_sparse_amd as ca
from oracle import chunk_attention_ref, chunk_attention_rows_ref, union_tables_ref

# Parity bars: bit-exact tables; attention within these bounds of the float64 oracle.
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
# LSE bounds.  Both kernels return lse = m * scale + log(l), where l sums the fp32
# exponentials before any rounding to bf16 (the bf16 path rounds the probabilities
# only for the P.V product), so no bf16 rounding reaches lse: only fp32 rounding
# does.
#  * Scores: fp32 accumulation of exact products of bf16 (or fp32) inputs.  Their
#    rounding grows with sum_d |q_d k_d|, which is of the order of the largest
#    logits and so of |lse|: about eight accumulations at 2^-24, rounded at
#    random, give a relative 2^-22; the bound takes 2^-20 of |lse|.
#  * Exponentials, the log and the two final roundings: a few fp32 ulps.
#  * The fp32 sum of the denominator: one add per staged block and row (up to
#    2048 at 128K), plus the split or piece merge.  Rounded at random its
#    relative error stays near sqrt(2048) * 2^-25 ~= 1.3e-6.
# The absolute term, 3e-5, is about twenty times that.  Measured: at most 3.8e-6
# on Gaussian inputs (|lse| < 12), 2.4e-4 where scaled keys put |lse| near 1340.
# A merge that weighted one split or piece wrong by 0.005% of the row's mass
# would already exceed the bound.  The fp32 path: 1e-5.
LSE_ABS = 3e-5
LSE_REL = 2.0 ** -20
F32_LSE_ABS = 1e-5


def check_lse(got, ref, what="lse", fp32=False):
    """got/ref: lse arrays of the same shape.  -inf exactly where the reference
    has no admissible key, elsewhere |got - ref| <= abs + 2^-20 |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    live = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), live), f"{what}: finite pattern differs"
    assert np.all(got[~live] == -np.inf) and np.all(ref[~live] == -np.inf), \
        f"{what}: non-finite entries other than -inf"
    if not live.any():
        return 0.0
    err = np.abs(got[live] - ref[live])
    bound = (F32_LSE_ABS if fp32 else LSE_ABS) + LSE_REL * np.abs(ref[live])
    ratio = float((err / bound).max())
    say(f"  {what}: lse max-abs {float(err.max()):.3e} (max |lse| {float(np.abs(ref[live]).max()):.2f}), "
        f"{ratio:.3f} of the bound")
    assert ratio <= 1.0, f"{what}: lse error {float(err.max())} exceeds its bound"
    return float(err.max())


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Dev:
    """Device copies of a workload's inputs."""

    def __init__(self, w: gen.Workload):
        self.w = w
        self.mask = torch.from_numpy(w.mask).cuda()
        self.q = w.q.cuda() if w.q is not None else None
        self.k = w.k.cuda() if w.k is not None else None
        self.v = w.v.cuda() if w.v is not None else None

    def tables(self):
        w = self.w
        return ca.build_union_tables(self.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)

    def attention(self, T, lens, k=None, v=None, return_lse=False):
        w = self.w
        return ca.chunk_attention(self.q, self.k if k is None else k, self.v if v is None else v,
                                  T, lens, w.prior, w.chunk, w.scale, return_lse=return_lse)


def oracle_tables(w):
    return union_tables_ref(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)


def oracle_full(w):
    T, ln = oracle_tables(w)
    q, k, v = (gen.tensor_to_f32(x) for x in (w.q, w.k, w.v))
    return chunk_attention_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale)


def oracle_full_parallel(w, arrays=None, workers=4):
    """oracle_full, run as independent slices: attention of KV group g of
    sequence b reads only that group's queries, cache rows and table, so each
    (b, g) slice goes through chunk_attention_ref on its own, on a few threads
    (NumPy's element-wise loops release the GIL; BLAS threads are shared out)."""
    import concurrent.futures as cf
    import os
    T, ln = oracle_tables(w)
    q, k, v = arrays if arrays is not None else f32_arrays(w)
    G = w.G
    O = np.zeros(q.shape, np.float32)
    lse = np.full(q.shape[:3], -np.inf, np.float32)

    def one(bg):
        b, g = bg
        sl = slice(b, b + 1)
        o, l_ = chunk_attention_ref(q[sl, g * G:(g + 1) * G], k[sl, g:g + 1], v[sl, g:g + 1],
                                    T[sl, g:g + 1], ln[sl, g:g + 1], w.prior[b:b + 1],
                                    w.chunk[b:b + 1], w.scale)
        O[b, g * G:(g + 1) * G] = o[0]
        lse[b, g * G:(g + 1) * G] = l_[0]

    jobs = [(b, g) for b in range(w.B) for g in range(w.H_kv)]
    n = max(1, min(workers, len(jobs)))
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=max(1, cores // n), user_api="blas")
    except Exception:  # threadpoolctl missing: BLAS keeps its own threads
        limit = None
    try:
        with cf.ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(one, jobs))
    finally:
        if limit is not None:
            limit.restore_original_limits()
    return O, lse


def f32_arrays(w):
    """Exact float32 copies of the workload's Q, K, V for the oracle."""
    return tuple(gen.tensor_to_f32(x) for x in (w.q, w.k, w.v))


def oracle_rows(w, rows, arrays=None):
    T, ln = oracle_tables(w)
    q, k, v = arrays if arrays is not None else f32_arrays(w)
    return chunk_attention_rows_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale, rows)


def sample_rows(w, seed=0, heads_per_group=2, extra=4):
    """Rows (b, h, i) covering first/last rows, tile and Q-block edges, every
    group, and some random rows."""
    rng = np.random.default_rng(seed)
    out = set()
    G = w.G
    for b in range(w.B):
        C = w.chunk[b]
        if C == 0:
            continue
        fixed = [0, 1, 31, 32, 63, 64, 95, C // 2, C - 33, C - 32, C - 2, C - 1]
        for g in range(w.H_kv):
            hs = rng.choice(np.arange(g * G, (g + 1) * G), size=min(heads_per_group, G),
                            replace=False)
            for h in hs:
                for i in fixed + [int(x) for x in rng.integers(0, C, extra)]:
                    if 0 <= i < C:
                        out.add((b, int(h), int(i)))
    return np.array(sorted(out), np.int64)


def compare_bf16(got, ref, what=""):
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    say(f"  {what}: max-abs {mx:.3e}  mean-abs {mean:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= BF16_MAX_ABS, f"{what}: max-abs {mx} > {BF16_MAX_ABS}"
    assert mean <= BF16_MEAN_ABS, f"{what}: mean-abs {mean} > {BF16_MEAN_ABS}"
    return mx, mean


# Unit roundoff of bf16: 8 significant bits, round to nearest even, so a rounded
# value moves by at most 2^-8 of itself.
U_BF16 = 2.0 ** -8


def oracle_full_absv(w):
    """The oracle's attention of |V| (same rows, tables and weights): for each
    output element, sum_t softmax(x)_t |V[t, d]|."""
    T, ln = oracle_tables(w)
    q, k, v = f32_arrays(w)
    return chunk_attention_ref(q, k, np.abs(v), T, ln, w.prior, w.chunk, w.scale)[0]


def check_bf16_rounding(got, ref, ref_absv, lse_ref, what=""):
    """Per-element bound of the bf16 path's roundings (every output element).

    The kernel forms p_t = exp(x_t - m) in fp32, rounds it to bf16 for the P.V
    product (p~_t = p_t (1 + r_t), |r_t| <= u = 2^-8), divides by the fp32 sum of
    the unrounded p_t and rounds O to bf16.  Against the exact result
    O* = sum_t p*_t v_t / sum_t p*_t that gives

      |O - O*| <= u |sum_t p_t r_t v_t| / l                 (P rounding)
                + u |O|                                      (output rounding)
                + 2 delta sum_t p_t |v_t| / l                (logit errors)
                <= u (A|V| + |O*|)(1 + 2^-7) + 2 delta A|V| + 1e-6,

    with A|V| = sum_t softmax(x)_t |v_t| (the oracle run on |V|, ``ref_absv``)
    and delta the logit error per key, taken at the row's lse bound
    (3e-5 + 2^-20 |lse|: both come from the fp32 score accumulation, which
    grows with the largest logits).  The fp32 accumulations of P.V and of the
    denominator add a few 2^-24 relative, inside the slack.  A worst case of
    the P rounding needs every r_t at u with the sign of v_t; it is what lets
    one dominant key with |v| near 5 reach about 2e-2.  Returns the largest
    ratio of error to bound."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    absv = np.asarray(ref_absv, np.float64)
    lse_ref = np.asarray(lse_ref, np.float64)
    delta = np.where(np.isfinite(lse_ref), LSE_ABS + LSE_REL * np.abs(lse_ref), 0.0)[..., None]
    bound = U_BF16 * (absv + np.abs(ref)) * (1 + 2.0 ** -7) + 2 * delta * absv + 1e-6
    err = np.abs(got - ref)
    ratio = err / bound
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    r = float(ratio[worst])
    say(f"  {what}: rounding-model bound, worst element at {tuple(int(x) for x in worst)}: "
        f"error {float(err[worst]):.3e}, bound {float(bound[worst]):.3e} ({r:.3f} of it); "
        f"median ratio {float(np.median(ratio)):.3f}")
    assert r <= 1.0, f"{what}: error {float(err[worst])} beyond the rounding bound {float(bound[worst])}"
    return r


# Block scores of the mask producer: each fp32 operand is split into bf16 hi + lo
# parts and a product taken as hi*hi + hi*lo + lo*hi on the bf16 matrix cores;
# what is left out (lo*lo and the two split residuals) is at most 3 * 2^-16 of
# |q_d k_d|, and the fp32 accumulation adds about 2^-19 of sum_d |q_d k_d|.
# The absolute term covers the pooling's fp32 error carried into the D products.
SCORE_ATOL = 2e-5
SCORE_REL = 2.0 ** -14


def score_bound(qbar_ref, kbar_ref):
    """Per-score bound of |GPU score - float64 score|, from the pooled operands:
    SCORE_ATOL + 2^-14 sum_d |qbar_d kbar_d|."""
    from oracle import block_scores_ref
    return SCORE_ATOL + SCORE_REL * block_scores_ref(np.abs(qbar_ref), np.abs(kbar_ref))


def check_scores(got, ref, bound, what="scores"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    ratio = float((np.abs(got - ref) / bound).max()) if got.size else 0.0
    say(f"  {what}: max |error| / bound {ratio:.3f}")
    assert ratio <= 1.0, f"{what}: score error beyond its bound ({ratio:.3f})"
    return ratio


def to_np(t: torch.Tensor) -> np.ndarray:
    return gen.tensor_to_f32(t.detach().cpu())
