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
# The bf16 path sums the bf16-rounded probabilities in the softmax denominator.
# bf16 carries 8 significant bits, so round-to-nearest-even leaves each within a
# relative 2^-8 of the exact value; log(l) is then within log(1 + 2^-8) ~= 3.9e-3
# of the exact LSE, plus fp32 rounding of the scores and the exponentials.
LSE_ABS = 4.5e-3


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


def to_np(t: torch.Tensor) -> np.ndarray:
    return gen.tensor_to_f32(t.detach().cpu())
