"""The per-element rounding bounds used by the GPU parity tests, checked on the
CPU against emulations of the GPU arithmetic (no GPU).

Attention outputs (``check_bf16_rounding``): the emulation takes the kernel's
roundings one by one: logits and exponentials in fp32, each probability
rounded to bf16 (round to nearest even) for the P.V product, the numerator and
the denominator (of the unrounded probabilities) summed in fp32, and the
quotient rounded to bf16.  Its outputs must sit inside the bound on every
element, for smooth and for peaky rows; a planted mistake (one P.V term
dropped, or a denominator 1% off) must not.

Block scores of the mask producer (``score_bound``): products of the bf16
hi / lo parts of fp32 values must sit inside the bound; with a cross term
dropped they must not.
"""
import numpy as np
import pytest

from tests.gpu_util import check_bf16_rounding, check_scores, score_bound


def _bf16_rne(x):
    """Round float32 values to the nearest bf16 value (ties to even), returned
    as float32."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16 << 16).astype(np.uint32).view(np.float32)


def _rows(seed, n_rows, n_keys, D, peak):
    rng = np.random.default_rng(seed)
    q = _bf16_rne(rng.standard_normal((n_rows, D)).astype(np.float32))
    k = rng.standard_normal((n_keys, D)).astype(np.float32)
    k[rng.integers(0, n_keys, 3)] *= peak  # a few keys that dominate their rows
    k = _bf16_rne(k)
    v = _bf16_rne(rng.standard_normal((n_keys, D)).astype(np.float32))
    return q, k, v, 1.0 / np.sqrt(D)


def _exact(q, k, v, scale):
    x = scale * (q.astype(np.float64) @ k.astype(np.float64).T)
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    l = e.sum(axis=1, keepdims=True)
    O = (e @ v.astype(np.float64)) / l
    absv = (e @ np.abs(v.astype(np.float64))) / l
    return O, absv, (m + np.log(l))[:, 0]


def _emulated(q, k, v, scale, drop_last=False, denom_scale=1.0):
    x = (np.float32(scale) * (q @ k.T)).astype(np.float32)
    m = x.max(axis=1, keepdims=True)
    p = np.exp(x - m).astype(np.float32)
    pr = _bf16_rne(p)
    if drop_last:
        pr[:, -1] = 0.0
    acc = (pr @ v).astype(np.float32)
    l = (p.sum(axis=1, dtype=np.float32, keepdims=True) * np.float32(denom_scale))
    return _bf16_rne((acc / l).astype(np.float32))


@pytest.mark.parametrize("peak", [1.0, 4.0, 12.0])
def test_emulated_bf16_path_is_inside_the_bound(peak):
    q, k, v, scale = _rows(3, 96, 512, 128, peak)
    O, absv, lse = _exact(q, k, v, scale)
    r = check_bf16_rounding(_emulated(q, k, v, scale), O, absv, lse, f"emulated, peak {peak}")
    assert r <= 1.0


@pytest.mark.parametrize("mistake", [dict(drop_last=True), dict(denom_scale=1.01)])
def test_planted_mistake_breaks_the_bound(mistake):
    q, k, v, scale = _rows(5, 96, 512, 128, 12.0)
    O, absv, lse = _exact(q, k, v, scale)
    with pytest.raises(AssertionError):
        check_bf16_rounding(_emulated(q, k, v, scale, **mistake), O, absv, lse, "planted")


# Block scores (``score_bound``): each fp32 pooled value is split into bf16 hi
# and lo parts, and a product is taken as hi*hi + hi*lo + lo*hi, accumulated
# in fp32.


def _split(x):
    hi = _bf16_rne(x)
    lo = _bf16_rne((x - hi).astype(np.float32))
    return hi, lo


def _split_scores(qbar, kbar, terms=("hl", "lh", "hh")):
    qh, ql = _split(qbar)
    kh, kl = _split(kbar)
    parts = {"hh": (qh, kh), "hl": (qh, kl), "lh": (ql, kh)}
    s = np.zeros(qbar.shape[:-1] + (kbar.shape[-2],), np.float32)
    for t in terms:  # products of bf16 values are exact in fp32
        a, b = parts[t]
        s = (s + np.einsum("bhqd,bhkd->bhqk", a.astype(np.float64), b.astype(np.float64))
             .astype(np.float32)).astype(np.float32)
    return s


def _pooled(seed, scale):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((1, 2, 32, 128)) * scale).astype(np.float32)
    k = (rng.standard_normal((1, 2, 96, 128)) * scale).astype(np.float32)
    return q, k


@pytest.mark.parametrize("scale", [0.125, 1.0, 8.0])
def test_split_scores_are_inside_the_bound(scale):
    q, k = _pooled(11, scale)
    ref = np.einsum("bhqd,bhkd->bhqk", q.astype(np.float64), k.astype(np.float64))
    check_scores(_split_scores(q, k), ref, score_bound(q, k), f"split scores, scale {scale}")


def test_split_scores_without_a_cross_term_break_the_bound():
    q, k = _pooled(13, 8.0)
    ref = np.einsum("bhqd,bhkd->bhqk", q.astype(np.float64), k.astype(np.float64))
    with pytest.raises(AssertionError):
        check_scores(_split_scores(q, k, terms=("hh", "hl")), ref, score_bound(q, k), "planted")
