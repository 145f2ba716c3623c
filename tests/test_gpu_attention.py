"""GPU parity of zero-copy paged chunk attention (through the C ABI) against
the float64 oracle.

* Small shapes (several tiles, ragged tails, C_max padding, D = 64 and 128,
  group sizes 1..8): every output element is compared.
* Full-size workloads: every output row of the 32K chunk, of the 128K chunk
  under each mask variant and of the ragged batch is compared with the oracle;
  at all 12 points of the vertical-slash sweep, sampled rows of every head are
  compared, and properties that hold at any size are checked on the whole
  output.
* Poison invariance: NaN in every unselected block and in the unused cache
  tail must leave O bit-identical (the kernel reads only the listed blocks).
* Closed forms: K = 0 with one-hot V gives exact per-block key counts; V = 1
  gives 1.
"""
import zlib

import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from tests.gpu_util import (BF16_MAX_ABS, F32_MAX_ABS, Dev, check_bf16_rounding, check_lse,
                            compare_bf16, oracle_full_absv,
                            f32_arrays, oracle_full, oracle_full_parallel, oracle_rows,
                            sample_rows, say, to_np)

pytestmark = pytest.mark.gpu


def _bern(p):
    return lambda rng, b, H, nq, pb: (rng.random((H, nq, pb)) < p).astype(np.uint8)


def _run(w, return_lse=True):
    d = Dev(w)
    T, lens = d.tables()
    out = d.attention(T, lens, return_lse=return_lse)
    torch.cuda.synchronize()
    return d, T, lens, out


# ----------------------------------------------------------------------------- fp32


def test_tiny_f32_full_parity():
    w = gen.make_workload("tiny_f32")
    say("tiny_f32 full parity")
    _, _, _, (O, lse) = _run(w)
    Or, lr = oracle_full(w)
    err = np.abs(to_np(O) - Or).max()
    say(f"  max-abs {err:.3e}")
    assert err <= F32_MAX_ABS
    check_lse(to_np(lse), lr, fp32=True)


@pytest.mark.parametrize("B,H_q,H_kv,D,prior,chunk,C_max", [
    (2, 4, 2, 128, (512, 1024), (192, 128), 200),
    (3, 2, 1, 64, (0, 64, 4096), (128, 64, 256), 256),
])
def test_f32_small_full_parity(B, H_q, H_kv, D, prior, chunk, C_max):
    w = gen.make_custom(B, H_q, H_kv, D, prior, chunk, "f32", 11, _bern(0.3), C_max=C_max)
    say(f"f32 B={B} H={H_q}/{H_kv} D={D} prior={prior} chunk={chunk}")
    _, _, _, (O, lse) = _run(w)
    Or, lr = oracle_full(w)
    assert np.abs(to_np(O) - Or).max() <= F32_MAX_ABS
    check_lse(to_np(lse), lr, fp32=True)


# ----------------------------------------------------------------------------- bf16 small


SMALL_BF16 = [
    # B, H_q, H_kv, D, prior, chunk, C_max
    (1, 4, 1, 128, (1024,), (256,), 256),
    (2, 8, 2, 128, (1024, 2048), (256, 128), 300),   # ragged chunk, C_max not a tile multiple
    (2, 8, 2, 64, (2048, 0), (192, 64), 192),        # D = 64, a sequence with no prior
    (1, 4, 4, 128, (640,), (320,), 320),             # G = 1
    (1, 16, 2, 128, (512,), (128,), 128),            # G = 8
    (2, 6, 2, 128, (256, 1536), (192, 256), 256),    # G = 3
    (8, 8, 1, 128, [64 * i for i in range(8)], [64] * 8, 64),  # B*H_kv = 8: XCD mapping
]


@pytest.mark.parametrize("B,H_q,H_kv,D,prior,chunk,C_max", SMALL_BF16)
def test_bf16_small_full_parity(B, H_q, H_kv, D, prior, chunk, C_max):
    w = gen.make_custom(B, H_q, H_kv, D, list(prior), list(chunk), "bf16", 21, _bern(0.2),
                        C_max=C_max)
    say(f"bf16 B={B} H={H_q}/{H_kv} D={D} prior={prior} chunk={chunk} C_max={C_max}")
    _, _, _, (O, lse) = _run(w)
    Or, lr = oracle_full(w)
    compare_bf16(to_np(O), Or, "O")
    check_bf16_rounding(to_np(O), Or, oracle_full_absv(w), lr, "O")
    live = np.isfinite(lr)
    assert np.array_equal(np.isfinite(to_np(lse)), live)
    check_lse(to_np(lse)[live], lr[live])
    for b in range(B):  # padding rows are exact zeros
        assert np.all(to_np(O)[b, :, chunk[b]:] == 0)


def test_bf16_dense_and_sparse_agree_on_dense_mask():
    # the all-ones mask run is the dense baseline: same as a table listing every block
    w = gen.make_custom(1, 8, 2, 128, [2048], [256], "bf16", 5, _bern(1.0))
    d = Dev(w)
    T, lens = d.tables()
    nkb = w.n_kv_blocks[0]
    Td = torch.full_like(T, -1)
    Td[..., :nkb] = torch.arange(nkb, dtype=torch.int32, device="cuda")
    ld = torch.full_like(lens, nkb)
    O1 = d.attention(T, lens)
    O2 = d.attention(Td, ld)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)


def test_bf16_deterministic_repeat():
    w = gen.make_custom(2, 8, 2, 128, [1024, 512], [256, 128], "bf16", 9, _bern(0.3))
    d = Dev(w)
    T, lens = d.tables()
    O1 = d.attention(T, lens).clone()
    O2 = d.attention(T, lens)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)


# ----------------------------------------------------------------------------- closed forms


def test_bf16_closed_form_one_hot_block_counts():
    # K = 0 makes every admissible key weigh exactly 1 (exp2(0)), so with
    # V_t = one_hot(t // 64) the output is the exact share of admissible keys per
    # block: it shows which blocks were read, including causal cut-offs.
    w = gen.make_custom(1, 8, 2, 64, [2048], [512], "bf16", 4, _bern(0.2))
    w.k.zero_()
    w.v.zero_()
    n_tok = w.prior[0] + w.chunk[0]
    assert n_tok // 64 <= w.D
    t = torch.arange(n_tok)
    w.v[0, :, t, t // 64] = 1.0
    _, _, _, (O, _) = _run(w)
    Or, _ = oracle_full(w)
    err = np.abs(to_np(O) - Or)
    # bf16 output rounding of a share in (0, 1]: relative 2^-8 (8 significant bits)
    assert np.all(err <= np.abs(Or) * 2.0 ** -8 + 1e-7)
    assert np.array_equal(to_np(O) != 0, Or != 0)


def test_bf16_closed_form_constant_values():
    w = gen.make_custom(1, 8, 2, 128, [4096], [256], "bf16", 6, _bern(0.3))
    w.v.fill_(1.0)
    _, _, _, (O, _) = _run(w)
    # the numerator sums the bf16-rounded probabilities and the denominator the
    # unrounded ones: each rounding is within 2^-8 relative, so O is within
    # 2^-8 of 1 (one bf16 step below 1); the roundings largely cancel, so
    # nearly every element is exactly 1
    Oh = to_np(O)
    assert np.all(np.abs(Oh - 1.0) <= 2.0 ** -8)
    assert np.mean(Oh == 1.0) >= 0.99


# ----------------------------------------------------------------------------- full sizes


_WL = {}


def _workload(name, **kw):
    """Full-size workloads; the 128K variants share Q/K/V (seed 1003) and differ in mask."""
    key = (name, tuple(sorted(kw.items())))
    if key in _WL:
        return _WL[key]
    if name in ("llama8b_128k", "vslash_128k"):
        base = _WL.get("base128")
        if base is None:
            base = gen.make_workload("llama8b_128k", variant="pairwise")
            _WL.clear()
            _WL["base128"] = base
            _WL["base128_f32"] = f32_arrays(base)
        w = gen.make_workload(name, with_tensors=False, **kw)
        w.q, w.k, w.v = base.q, base.k, base.v
        w.meta["arrays"] = _WL["base128_f32"]
    else:
        _WL.clear()
        w = gen.make_workload(name, **kw)
        w.meta["arrays"] = f32_arrays(w)
    _WL[key] = w
    return w


# Whole-output parity: every output row of the 32K chunk, of every 128K mask
# variant and of the ragged batch is compared with the oracle.
WHOLE = [
    ("llama8b_32k", {}),
    ("llama8b_128k", dict(variant="pairwise")),
    ("llama8b_128k", dict(variant="colshared")),
    ("llama8b_128k", dict(variant="groupshared")),
    ("llama8b_128k", dict(variant="dense")),
    ("ragged_b4", {}),
]


def _whole_output_properties(w, d, O):
    # finite everywhere, padding rows zero, bounded by max|V| (a convex combination)
    assert bool(torch.isfinite(O).all())
    assert float(O.abs().max()) <= float(d.v.abs().max())
    for b in range(w.B):
        assert bool((O[b, :, w.chunk[b]:] == 0).all())


@pytest.mark.parametrize("name,kw", WHOLE)
def test_full_size_whole_output_parity(name, kw):
    say(f"full-size {name} {kw}: generating")
    w = _workload(name, **kw)
    d = Dev(w)
    T, lens = d.tables()
    O, lse = d.attention(T, lens, return_lse=True)
    torch.cuda.synchronize()
    say(f"  union sum len {int(lens.sum())}; oracle over every row")
    Or, lr = oracle_full_parallel(w, arrays=w.meta["arrays"])
    compare_bf16(to_np(O), Or, f"all {w.B * w.H_q * w.C_max} rows")
    check_lse(to_np(lse), lr)
    if name == "llama8b_32k":  # every element against the rounding model (oracle on |V|)
        q, k, v = w.meta["arrays"]
        absv, _ = oracle_full_parallel(w, arrays=(q, k, np.abs(v)))
        check_bf16_rounding(to_np(O), Or, absv, lr, "all rows")
    _whole_output_properties(w, d, O)


VSLASH = [(dn, hm) for dn in gen.VSLASH_DENSITIES for hm in ("identical", "independent")]


@pytest.mark.parametrize("density,heads", VSLASH)
def test_vslash_sampled_parity(density, heads):
    # every point of the structured-mask sweep: rows of all four heads of every
    # group at tile and Q-block edges plus random rows
    kw = dict(density=density, heads=heads)
    say(f"vslash_128k {kw}: generating")
    w = _workload("vslash_128k", **kw)
    d = Dev(w)
    T, lens = d.tables()
    O, lse = d.attention(T, lens, return_lse=True)
    torch.cuda.synchronize()
    say(f"  union sum len {int(lens.sum())}")
    rows = sample_rows(w, seed=zlib.crc32(repr(kw).encode()) % 1000, heads_per_group=w.G,
                       extra=8)
    Or, lr = oracle_rows(w, rows, arrays=w.meta["arrays"])
    r = torch.from_numpy(rows).cuda()
    compare_bf16(to_np(O[r[:, 0], r[:, 1], r[:, 2]]), Or, f"{len(rows)} sampled rows")
    check_lse(to_np(lse[r[:, 0], r[:, 1], r[:, 2]]), lr)
    _whole_output_properties(w, d, O)


@pytest.mark.parametrize("name,kw", [
    ("llama8b_128k", dict(variant="colshared")),
    ("ragged_b4", {}),
])
def test_full_size_poison_invariance(name, kw):
    say(f"poison {name} {kw}")
    w = _workload(name, **kw)
    d = Dev(w)
    T, lens = d.tables()
    O = d.attention(T, lens)
    nblk = w.L // 64 + 1
    sel = torch.zeros((w.B, w.H_kv, nblk), dtype=torch.bool, device="cuda")
    Tc = torch.where(T >= 0, T, torch.full_like(T, nblk - 1)).long()
    sel.scatter_(2, Tc, True)
    sel[..., nblk - 1] = False
    tok = torch.arange(w.L, device="cuda")
    keep = sel[:, :, tok // 64]
    for b in range(w.B):
        keep[b, :, w.prior[b] + w.chunk[b]:] = False
    kp = d.k.clone()
    vp = d.v.clone()
    kp[~keep] = float("nan")
    vp[~keep] = float("nan")
    say(f"  poisoned {float((~keep).float().mean()):.3f} of the cache rows")
    O2 = d.attention(T, lens, k=kp, v=vp)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
    del kp, vp


def test_long_table_beyond_entry_list():
    # More plain table entries (about 4350) than the kernel's LDS entry list
    # holds (4096): those workgroups walk T itself.  Split-KV cuts the same
    # long table into ranges.
    w = gen.make_custom(1, 8, 2, 128, [4352 * 64], [192], "bf16", 41, _bern(0.6))
    say(f"long table: prior {w.prior[0]}, L {w.L}")
    d = Dev(w)
    T, lens = d.tables()
    say(f"  lens {lens.tolist()}")
    assert int(lens.min()) > 4096
    O, lse = d.attention(T, lens, return_lse=True)
    Os, lses = ca.chunk_attention(d.q, d.k, d.v, T, lens, w.prior, w.chunk, w.scale,
                                  return_lse=True, n_splits=4)
    torch.cuda.synchronize()
    rows = sample_rows(w, seed=41)
    Or, lr = oracle_rows(w, rows)
    r = torch.from_numpy(rows).cuda()
    for name, (o, l) in (("no split", (O, lse)), ("4 splits", (Os, lses))):
        compare_bf16(to_np(o[r[:, 0], r[:, 1], r[:, 2]]), Or, f"{name}, {len(rows)} rows")
        check_lse(to_np(l[r[:, 0], r[:, 1], r[:, 2]]), lr)
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(Os).all())


# ----------------------------------------------------------------------------- errors


def test_binding_rejects_bad_arguments():
    w = gen.make_custom(1, 4, 1, 128, [1024], [128], "bf16", 1, _bern(0.2))
    d = Dev(w)
    T, lens = d.tables()
    with pytest.raises(ValueError):
        ca.chunk_attention(d.q.float(), d.k, d.v, T, lens, w.prior, w.chunk)
    with pytest.raises(ValueError):
        ca.chunk_attention(d.q, d.k, d.v, T.cpu(), lens, w.prior, w.chunk)
    with pytest.raises(ca.CompactAttnError) as e:
        ca.chunk_attention(d.q, d.k, d.v, T, lens, [1000], w.chunk)
    assert e.value.status == 4
    with pytest.raises(ca.CompactAttnError) as e:
        ca.chunk_attention(d.q, d.k, d.v, T, lens, [1024], [192])  # chunk > C_max
    assert e.value.status == 2


# ----------------------------------------------------------------------------- rare paths


@pytest.mark.parametrize("D,growth", [(128, 0.35), (64, 0.5), (128, -0.03)])
def test_bf16_running_max_moves(D, growth):
    # Keys scaled by (1 + growth * block): with growth > 0 later blocks keep raising
    # the row max past the kernel's rescale threshold, so the path that folds the
    # pending P.V in early and rescales runs many times; growth < 0 never moves it.
    w = gen.make_custom(2, 8, 2, D, [2048, 1024], [192, 128], "bf16", 31, _bern(0.5),
                        C_max=192)
    n_blk = w.L // 64
    scale = (1.0 + growth * torch.arange(n_blk, dtype=torch.float32)).clamp_min(0.2)
    w.k.copy_((w.k.float().view(w.B, w.H_kv, n_blk, 64, D) * scale.view(1, 1, n_blk, 1, 1))
              .view_as(w.k).to(torch.bfloat16))
    say(f"running max moves: D={D} growth={growth}")
    _, _, _, (O, lse) = _run(w)
    Or, lr = oracle_full(w)
    compare_bf16(to_np(O), Or, "O")
    check_bf16_rounding(to_np(O), Or, oracle_full_absv(w), lr, "O")
    live = np.isfinite(lr)
    check_lse(to_np(lse)[live], lr[live])


@pytest.mark.parametrize("D", [128, 64])
def test_bf16_logit_spikes(D):
    # A few blocks with keys scaled by 300 (logits far past the fp32 range of an
    # exponential taken against the earlier running max) and some by 20, in the
    # middle of the tables: the running max jumps by hundreds of log2 units at
    # once, and by a few units elsewhere.
    w = gen.make_custom(2, 8, 2, D, [2048, 1024], [192, 128], "bf16", 47, _bern(0.6),
                        C_max=192)
    n_blk = w.L // 64
    scale = torch.ones(n_blk)
    scale[[5, 17, 26]] = 300.0
    scale[[3, 9, 12, 21]] = 20.0
    w.k.copy_((w.k.float().view(w.B, w.H_kv, n_blk, 64, D) * scale.view(1, 1, n_blk, 1, 1))
              .view_as(w.k).to(torch.bfloat16))
    say(f"logit spikes: D={D}")
    _, _, _, (O, lse) = _run(w)
    Or, lr = oracle_full(w)
    compare_bf16(to_np(O), Or, "O")
    check_bf16_rounding(to_np(O), Or, oracle_full_absv(w), lr, "O")
    live = np.isfinite(lr)
    check_lse(to_np(lse)[live], lr[live])


def test_bf16_junk_table_entries_are_skipped():
    # Entries outside [0, n_kv_blocks) anywhere in T, and len past NKB_max, are never
    # dereferenced: the output equals the run on the clean table bit for bit.
    w = gen.make_custom(2, 8, 2, 128, [1024, 512], [128, 128], "bf16", 17, _bern(0.3),
                        NKB_max=40)
    d = Dev(w)
    T, lens = d.tables()
    O = d.attention(T, lens).clone()
    Tj = T.clone()
    lj = lens.clone()
    for b in range(w.B):
        for g in range(w.H_kv):
            n = int(lens[b, g])
            row = T[b, g, :n].tolist()
            junk = [-5] + row[:n // 2] + [10 ** 6, -1] + row[n // 2:] + [w.n_kv_blocks[b]]
            Tj[b, g, :] = -1
            Tj[b, g, :len(junk)] = torch.tensor(junk, dtype=torch.int32)
            lj[b, g] = 10 ** 6 if (b + g) % 2 else len(junk)
    O2 = d.attention(Tj, lj)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
