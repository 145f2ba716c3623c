"""GPU parity of the explicit-compaction baseline (through the C ABI).

CompactAttention, abstract: the tables let attention read selected KV blocks
in place; compacting them first is the copy this avoids.  The compaction call
must (a) produce the oracle's destination table exactly, (b) copy every
selected block bit-exactly to its destination, and (c) leave the attention
result bit-identical to zero-copy execution on the original cache, even with
NaN in every block of the output buffers that the copy does not write.
"""
import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from oracle import compact_kv_ref
from tests.gpu_util import Dev, oracle_tables, say, to_np

pytestmark = pytest.mark.gpu


def _bern(p):
    return lambda rng, b, H, nq, pb: (rng.random((H, nq, pb)) < p).astype(np.uint8)


def _check(w):
    d = Dev(w)
    T, lens = d.tables()
    O0, l0 = d.attention(T, lens, return_lse=True)
    k_out = torch.full_like(d.k, float("nan"))
    v_out = torch.full_like(d.v, float("nan"))
    k_out, v_out, T_out = ca.compact_kv(d.k, d.v, T, lens, w.prior, w.chunk, k_out, v_out)
    O1, l1 = d.attention(T_out, lens, k=k_out, v=v_out, return_lse=True)
    torch.cuda.synchronize()
    # (a) destination table, against the oracle on the oracle's own tables
    Tr, lr = oracle_tables(w)
    k = gen.tensor_to_f32(w.k)
    v = gen.tensor_to_f32(w.v)
    kr, vr, Tor, written = compact_kv_ref(k, v, Tr, lr, w.prior, w.chunk)
    np.testing.assert_array_equal(T_out.cpu().numpy(), Tor)
    # (b) copied blocks, bit-exact (values are exact in float32)
    wmask = torch.from_numpy(written).cuda()
    rows = wmask.repeat_interleave(64, dim=2)[:, :, :w.L]
    say(f"  {w.name}: {int(written.sum())} blocks copied")
    np.testing.assert_array_equal(to_np(k_out[rows]), kr[rows.cpu().numpy()])
    np.testing.assert_array_equal(to_np(v_out[rows]), vr[rows.cpu().numpy()])
    # (c) attention over the compact buffer equals zero-copy attention exactly
    assert torch.equal(O0, O1)
    assert torch.equal(l0, l1)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_compact_small(dtype, D):
    w = gen.make_custom(B=3, H_q=8, H_kv=2, D=D, prior=[1920, 0, 4096], chunk=[384, 256, 192],
                        C_max=448, dtype=dtype, seed=77 + D, cell_fn=_bern(0.15),
                        name=f"compact_small_{dtype}_{D}")
    say(f"compact small {dtype} D={D}")
    _check(w)


def test_compact_empty_tables():
    # all-zero prior mask and no triangle: every table is empty, nothing copied
    w = gen.make_custom(B=1, H_q=4, H_kv=1, D=128, prior=[1024], chunk=[128], dtype="bf16",
                        seed=5, cell_fn=_bern(0.0), triangle=False, name="compact_empty")
    say("compact empty tables")
    _check(w)


def test_compact_full_size_32k():
    w = gen.make_workload("llama8b_32k")
    say("compact llama8b_32k")
    _check(w)


@pytest.mark.parametrize("seed", range(16))
def test_compact_fuzz(seed):
    # seeded random batch, heads, head dim, element type, ragged prior / chunk
    # lengths (zero included), padding and mask density
    rng = np.random.default_rng(50_000 + seed)
    H_kv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 5))
    D = int(rng.choice([64, 128]))
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    prior = [64 * int(rng.integers(0, 40)) for _ in range(B)]
    chunk = [64 * int(rng.integers(0, 5)) for _ in range(B)]
    if max(chunk) == 0:
        chunk[0] = 64
    C_max = max(chunk) + 64 * int(rng.integers(0, 2))
    p = float(rng.choice([0.0, 0.1, 0.5, 1.0]))
    w = gen.make_custom(B, G * H_kv, H_kv, D, prior, chunk, dtype, 60_000 + seed, _bern(p),
                        C_max=C_max, name=f"compact_fuzz{seed}")
    say(f"compact fuzz {seed}: B={B} H={G * H_kv}/{H_kv} D={D} {dtype} prior={prior} "
        f"chunk={chunk} p={p}")
    _check(w)
