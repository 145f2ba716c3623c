"""GPU parity of balanced chunk attention (ca_chunk_attention_balanced).

A planning kernel cuts the longest per-tile table walks into pieces and lists
every piece longest first; the pieces run, and cut tiles are merged.  Checked
here:
* outputs and LSE against the float64 oracle (full at small sizes, sampled
  rows at 128K), on uneven per-group tables and on one GPU's tensor-parallel
  share (one KV head, so every tile is cut);
* bit-identical output to ca_chunk_attention where the walks already balance
  (nothing cut: the same kernel arithmetic);
* the plan read back from the workspace: every tile's pieces listed exactly
  once, piece counts consistent, size classes non-increasing, the count within
  the launch grid;
* NaN outside the selected blocks changes nothing; one workspace serves calls
  of different shapes in a row; fp32 runs the unplanned kernel;
* more tiles than the planner keeps in LDS (its walks then pass through the
  workspace).
"""
import zlib

import numpy as np
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from tests.gpu_util import (F32_MAX_ABS, check_lse, Dev, compare_bf16, oracle_full, oracle_rows,
                            sample_rows, say, to_np)

pytestmark = pytest.mark.gpu

MAX_PIECES = 8
PLAN_MAX_SLOTS = 1024


def _bern(p):
    return lambda rng, b, H, nq, pb: (rng.random((H, nq, pb)) < p).astype(np.uint8)


def _by_group(dens, G):
    """Mask density per KV group (the heads of group g draw with dens[g])."""
    def fn(rng, b, H, nq, pb):
        p = np.repeat(np.asarray(dens, np.float64), G)[:H, None, None]
        return (rng.random((H, nq, pb)) < p).astype(np.uint8)
    return fn


def _balanced(d, T, lens, ws=None, return_lse=True):
    w = d.w
    return ca.chunk_attention(d.q, d.k, d.v, T, lens, w.prior, w.chunk, w.scale,
                              return_lse=return_lse, balanced=True, workspace=ws)


def _n_t(w):
    return (w.G * ((w.C_max + 31) // 32) + 7) // 8


def _read_plan(ws, w):
    """(count, items [count, 4] of (b*H_kv+g, tile, piece, pieces), pieces per tile)."""
    rows = w.B * w.H_q * w.C_max
    units = w.B * w.H_kv * _n_t(w)
    plan_off = MAX_PIECES * rows * w.D * 4 + MAX_PIECES * rows * 2 * 4
    plan_bytes = (4 + 4 * (units + 2 * PLAN_MAX_SLOTS)) * 4
    pieces_off = plan_off + (plan_bytes + 15) // 16 * 16
    ints = ws.cpu().view(torch.int32).numpy()
    count = int(ints[plan_off // 4])
    items = ints[plan_off // 4 + 4: plan_off // 4 + 4 + 4 * count].reshape(-1, 4)
    return count, items, ints[pieces_off // 4: pieces_off // 4 + units]


def _walks(w, T, lens):
    """The planner's measure of each 8-wave tile's work: the table's entries
    less the chunk blocks above the last block the tile's rows may see (exact
    when the chunk's causal block triangle is selected, as here)."""
    Th, lh = T.cpu().numpy(), lens.cpu().numpy()
    n_t, n_pb = _n_t(w), (w.C_max + 31) // 32
    out = np.zeros((w.B, w.H_kv, n_t), np.int64)
    for b in range(w.B):
        P, C = w.prior[b], w.chunk[b]
        nkb = (P + C + 63) // 64
        for t in range(n_t):
            if (t * 8) // w.G * 32 >= C:
                continue
            last_pb = min((t * 8 + 7) // w.G, n_pb - 1)
            kb_limit = (P + min(C, (last_pb + 1) * 32) - 1) // 64
            for g in range(w.H_kv):
                row = Th[b, g, :lh[b, g]]
                walk = int(np.searchsorted(row, kb_limit, side="right"))
                out[b, g, t] = max(int(lh[b, g]) - (nkb - 1 - kb_limit), 0)
                assert out[b, g, t] == walk  # every chunk block is in the table
    return out.reshape(-1)


def _check_plan(ws, w, T, lens):
    count, items, pieces = _read_plan(ws, w)
    n_t = _n_t(w)
    units = w.B * w.H_kv * n_t
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert 1 <= count <= units + 2 * min(cus, PLAN_MAX_SLOTS)
    assert np.all((pieces >= 1) & (pieces <= MAX_PIECES))
    assert int(pieces.sum()) == count
    want = sorted((u, t, k) for u in range(w.B * w.H_kv) for t in range(n_t)
                  for k in range(int(pieces[u * n_t + t])))
    assert sorted(map(tuple, items[:, :3].tolist())) == want
    assert np.all(items[:, 3] == pieces[items[:, 0] * n_t + items[:, 1]])
    walk = _walks(w, T, lens)
    wmax = int(walk.max())
    n = items[:, 3]
    wu = walk[items[:, 0] * n_t + items[:, 1]]
    size = wu * (items[:, 2] + 1) // n - wu * items[:, 2] // n
    cls = np.minimum(63, size // (wmax // 64 + 1))  # the planner's 64 size classes
    assert np.all(np.diff(cls) <= 0), "pieces not listed longest first"
    return pieces


SHAPES = [
    # B, H_q, H_kv, D, prior, chunk, C_max, per-group densities
    (1, 8, 2, 128, [4096], [512], 512, [1.0, 0.05]),
    (2, 16, 4, 128, [4096, 1024], [512, 256], 512, [1.0, 0.05, 0.3, 0.0]),
    (3, 8, 1, 64, [1920, 0, 4096], [384, 256, 192], 448, [0.2]),
    (2, 4, 4, 64, [6144, 640], [128, 64], 192, [0.5, 0.0, 1.0, 0.02]),
]


@pytest.mark.parametrize("B,H_q,H_kv,D,prior,chunk,C_max,dens", SHAPES)
def test_balanced_small_full_parity(B, H_q, H_kv, D, prior, chunk, C_max, dens):
    w = gen.make_custom(B, H_q, H_kv, D, prior, chunk, "bf16", 300 + sum(prior) % 97,
                        _by_group(dens, H_q // H_kv), C_max=C_max, name="balanced_small")
    say(f"balanced small B={B} H={H_q}/{H_kv} D={D} prior={prior} chunk={chunk} dens={dens}")
    d = Dev(w)
    T, lens = d.tables()
    ws = torch.empty(ca.balanced_workspace_size(B, H_q, H_kv, C_max, D), dtype=torch.uint8,
                     device="cuda")
    O, lse = _balanced(d, T, lens, ws)
    torch.cuda.synchronize()
    pieces = _check_plan(ws, w, T, lens)
    say(f"  tiles {pieces.size}, pieces {int(pieces.sum())}, cut tiles {int((pieces > 1).sum())}")
    assert (pieces > 1).any()  # small grids: tiles are cut to fill the compute units
    Or, lr = oracle_full(w)
    compare_bf16(to_np(O), Or, "O")
    live = np.isfinite(lr)
    gl = to_np(lse)
    assert np.array_equal(np.isfinite(gl), live)
    check_lse(gl[live], lr[live])
    for b in range(B):
        assert bool((O[b, :, chunk[b]:] == 0).all())


def test_balanced_equals_plain_when_even():
    # dense tables of equal length: the walks already balance, nothing is cut,
    # and the planned kernel does the plain kernel's arithmetic
    if torch.cuda.get_device_properties(0).multi_processor_count > 256:
        pytest.skip("the plain kernel takes 8-wave workgroups here only up to 256 CUs")
    w = gen.make_custom(1, 32, 8, 128, [8192], [2048], "bf16", 41,
                        lambda rng, b, H, nq, pb: np.ones((H, nq, pb), np.uint8),
                        name="balanced_even")
    say("balanced == plain on even tables")
    d = Dev(w)
    T, lens = d.tables()
    ws = torch.empty(ca.balanced_workspace_size(1, 32, 8, 2048, 128), dtype=torch.uint8,
                     device="cuda")
    Ob, lb = _balanced(d, T, lens, ws)
    Op, lp = d.attention(T, lens, return_lse=True)
    torch.cuda.synchronize()
    pieces = _check_plan(ws, w, T, lens)
    assert np.all(pieces == 1)
    assert torch.equal(Ob, Op)
    assert torch.equal(lb, lp)


@pytest.mark.parametrize("variant", ["pairwise", "colshared"])
def test_balanced_tp_shard_128k_sampled(variant):
    # one GPU's share of the 128K chunk: one KV head, 32 tiles, each cut
    from tests.test_gpu_split import _tp_shard
    say(f"balanced tp-shard 128K {variant}")
    w = _tp_shard(variant)
    d = Dev(w)
    T, lens = d.tables()
    ws = torch.empty(ca.balanced_workspace_size(1, 4, 1, 2048, 128), dtype=torch.uint8,
                     device="cuda")
    O, lse = _balanced(d, T, lens, ws)
    torch.cuda.synchronize()
    pieces = _check_plan(ws, w, T, lens)
    assert pieces.min() > 1
    rows = sample_rows(w, seed=zlib.crc32(variant.encode()) % 1000, heads_per_group=4, extra=16)
    Or, lr = oracle_rows(w, rows)
    r = torch.from_numpy(rows).cuda()
    compare_bf16(to_np(O[r[:, 0], r[:, 1], r[:, 2]]), Or, f"{len(rows)} sampled rows")
    check_lse(to_np(lse[r[:, 0], r[:, 1], r[:, 2]]), lr)
    assert bool(torch.isfinite(O).all())


def test_balanced_poison_and_workspace_reuse():
    # NaN in every cache row outside the selected blocks changes nothing; the
    # same workspace then serves a smaller call
    w = gen.make_custom(1, 8, 2, 128, [16384], [512], "bf16", 78, _by_group([0.3, 0.02], 4),
                        name="balanced_poison")
    say("balanced poison invariance and workspace reuse")
    d = Dev(w)
    T, lens = d.tables()
    ws = torch.empty(ca.balanced_workspace_size(1, 8, 2, 512, 128), dtype=torch.uint8,
                     device="cuda")
    O = _balanced(d, T, lens, ws, return_lse=False).clone()
    Th, lh = T.cpu().numpy(), lens.cpu().numpy()
    keep = np.zeros((w.B, w.H_kv, w.L), bool)
    for g in range(w.H_kv):
        for kb in Th[0, g, :lh[0, g]]:
            keep[0, g, kb * 64:(kb + 1) * 64] = True
    km = torch.from_numpy(~keep).cuda()
    kp, vp = d.k.clone(), d.v.clone()
    kp[km] = float("nan")
    vp[km] = float("nan")
    O2 = ca.chunk_attention(d.q, kp, vp, T, lens, w.prior, w.chunk, w.scale, balanced=True,
                            workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
    w2 = gen.make_custom(2, 4, 1, 128, [1024, 256], [128, 64], "bf16", 79, _bern(0.4),
                         C_max=128, name="balanced_second")
    d2 = Dev(w2)
    T2, l2 = d2.tables()
    O3, lse3 = _balanced(d2, T2, l2, ws)
    torch.cuda.synchronize()
    Or, lr = oracle_full(w2)
    compare_bf16(to_np(O3), Or, "second call")
    live = np.isfinite(lr)
    check_lse(to_np(lse3)[live], lr[live])


def test_balanced_fp32_runs_plain_kernel():
    w = gen.make_custom(2, 8, 2, 64, [1024, 512], [256, 128], "f32", 80, _bern(0.3), C_max=256,
                        name="balanced_f32")
    say("balanced fp32")
    d = Dev(w)
    T, lens = d.tables()
    Ob, lb = _balanced(d, T, lens)
    Op, lp = d.attention(T, lens, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(Ob, Op) and torch.equal(lb, lp)
    Or, _ = oracle_full(w)
    assert float(np.abs(to_np(Ob) - Or).max()) <= F32_MAX_ABS


def test_balanced_many_tiles_plan_in_global_scratch():
    # more tiles (B * H_kv * tiles per group = 17 * 8 * 64) than the planner
    # keeps in LDS: the walks go through the pieces array between its passes
    B, H_q, H_kv, D, C_max = 17, 64, 8, 64, 2048
    rng = np.random.default_rng(91)
    prior = [64 * int(x) for x in rng.integers(0, 12, B)]
    chunk = [64 * int(x) for x in rng.integers(1, 33, B)]
    chunk[0] = C_max
    w = gen.make_custom(B, H_q, H_kv, D, prior, chunk, "bf16", 92,
                        _by_group([1.0, 0.1, 0.5, 0.0, 0.3, 1.0, 0.05, 0.7], H_q // H_kv),
                        C_max=C_max, name="balanced_many_tiles")
    assert B * H_kv * _n_t(w) > 8192
    say(f"balanced with {B * H_kv * _n_t(w)} tiles")
    d = Dev(w)
    T, lens = d.tables()
    ws = torch.empty(ca.balanced_workspace_size(B, H_q, H_kv, C_max, D), dtype=torch.uint8,
                     device="cuda")
    O, lse = _balanced(d, T, lens, ws)
    torch.cuda.synchronize()
    _check_plan(ws, w, T, lens)
    rows = sample_rows(w, seed=93, heads_per_group=1, extra=2)
    Or, lr = oracle_rows(w, rows)
    r = torch.from_numpy(rows).cuda()
    compare_bf16(to_np(O[r[:, 0], r[:, 1], r[:, 2]]), Or, f"{len(rows)} sampled rows")
    check_lse(to_np(lse[r[:, 0], r[:, 1], r[:, 2]]), lr)
    for b in range(B):
        assert bool((O[b, :, chunk[b]:] == 0).all())
