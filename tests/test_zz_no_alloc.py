"""ca_chunk_attention_split_noalloc through the C ABI: split-KV attention whose
partials live in the library's static device array, for callers that cannot
allocate.  Its output must equal ca_chunk_attention_split's (same kernels, a
caller workspace) bit for bit, and both must stay within the parity bounds of
the float64 oracle.  Two calls in a row share the array: the second, on a
smaller input, finds the first call's partials there and must not see them.
"""
import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from tests.gpu_util import (F32_MAX_ABS, Dev, check_lse, compare_bf16, oracle_full, say,
                            to_np)

pytestmark = pytest.mark.gpu


def _bern(p):
    return lambda rng, b, H, nq, pb: (rng.random((H, nq, pb)) < p).astype(np.uint8)


def _noalloc_vs_split(w, n_splits):
    d = Dev(w)
    T, lens = d.tables()
    out = torch.full_like(d.q, float("nan"))
    lse = torch.full((w.B, w.H_q, w.C_max), float("nan"), dtype=torch.float32, device="cuda")
    ca.chunk_attention_split_noalloc(d.q, d.k, d.v, T, lens, w.prior, w.chunk, n_splits,
                                     w.scale, out=out, lse=lse)
    ws = torch.empty(ca.workspace_size(w.B, w.H_q, w.C_max, w.D, n_splits), dtype=torch.uint8,
                     device="cuda")
    ref_o, ref_l = ca.chunk_attention(d.q, d.k, d.v, T, lens, w.prior, w.chunk, w.scale,
                                      return_lse=True, n_splits=n_splits, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o), "no-alloc output differs from the workspace split's"
    assert torch.equal(lse, ref_l), "no-alloc lse differs from the workspace split's"
    Or, lr = oracle_full(w)
    if w.dtype == "bf16":
        compare_bf16(to_np(out), Or, f"O, {n_splits} splits")
    else:
        err = float(np.abs(to_np(out) - Or).max())
        say(f"  O, {n_splits} splits: max-abs {err:.3e}")
        assert err <= F32_MAX_ABS
    check_lse(to_np(lse), lr, f"lse, {n_splits} splits", fp32=w.dtype == "f32")
    for b in range(w.B):
        assert bool((out[b, :, w.chunk[b]:] == 0).all())


def test_noalloc_two_calls_second_smaller():
    # one GPU's tensor-parallel share of a 2048-token chunk over a 16K prior
    # (8 splits: 32.5 MiB of the array), then a ragged D = 64 batch (4 splits)
    big = gen.make_custom(1, 4, 1, 128, [16384], [2048], "bf16", 71, _bern(0.3))
    say(f"no-alloc call 1: {big.B}x{big.H_q}/{big.H_kv} D={big.D} prior {big.prior} "
        f"chunk {big.chunk}, 8 splits")
    _noalloc_vs_split(big, 8)
    small = gen.make_custom(2, 8, 2, 64, [1024, 512], [256, 128], "bf16", 72, _bern(0.4),
                            C_max=256)
    say(f"no-alloc call 2: {small.B}x{small.H_q}/{small.H_kv} D={small.D} prior {small.prior} "
        f"chunk {small.chunk}, 4 splits")
    _noalloc_vs_split(small, 4)


def test_noalloc_fp32_and_refusal():
    w = gen.make_custom(1, 4, 1, 64, [1024], [256], "f32", 73, _bern(0.25))
    say("no-alloc fp32: tiny shape, 8 splits")
    _noalloc_vs_split(w, 8)
    # a split past the array's size is refused and writes nothing
    big = gen.make_custom(1, 32, 8, 128, [2048], [2048], "bf16", 74, _bern(0.2))
    d = Dev(big)
    T, lens = d.tables()
    out = torch.zeros_like(d.q)
    with pytest.raises(ca.CompactAttnError) as e:
        ca.chunk_attention_split_noalloc(d.q, d.k, d.v, T, lens, big.prior, big.chunk, 2,
                                         big.scale, out=out)
    assert e.value.status == 6
    torch.cuda.synchronize()
    assert bool((out == 0).all())
