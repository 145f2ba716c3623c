"""GPU parity of balanced chunk attention (ca_chunk_attention_balanced).

One workgroup per compute unit ("slot"); each derives the same plan from the
table lengths: slot s first runs tile s (whole, or its first A work units, A
the even share), then the tails of the cut tiles, laid end to end over the
slots' spare capacity.  A cut tile's pieces write partials, which a second
kernel merges.  Checked here:
* outputs and LSE against the float64 oracle (full at small sizes, sampled
  rows at 128K), on uneven per-group tables and on one GPU's tensor-parallel
  share (one KV head: every tile is cut into many pieces);
* the pieces of every tile, read back from the part numbering the kernel
  leaves in the workspace, against a model of the plan written here from its
  description;
* bit-identical output to ca_chunk_attention where the walks already balance
  (nothing cut: the same kernel arithmetic);
* NaN outside the selected blocks changes nothing; one workspace serves calls
  of different shapes in a row and a workspace of garbage bytes works; a
  captured graph replayed between eager calls matches the eager result; fp32 and shapes with more tiles than compute
  units run the plain kernel.
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

PLAN_MAX_SLOTS = 1024   # slots the workspace is sized for
BAL_MIN_SHARE = 32      # least work units per slot
JOB_COST = 12           # work units the plan counts per job


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


def _workspace(w, zero=True):
    n = ca.balanced_workspace_size(w.B, w.H_q, w.H_kv, w.C_max, w.D)
    return (torch.zeros if zero else torch.empty)(n, dtype=torch.uint8, device="cuda")


def _part_numbering(ws, w):
    """The plan's part numbering (tiles + 1 ints, plan order) from the workspace."""
    units = w.B * w.H_kv * _n_t(w)
    parts = 2 * units + PLAN_MAX_SLOTS
    up16 = lambda x: (x + 15) // 16 * 16
    off = up16(up16(parts * 256 * w.D * 4) + parts * 256 * 2 * 4)
    return ws[off: off + 4 * (units + 1)].cpu().numpy().view(np.int32).astype(np.int64)


def _plan_tiles(w):
    """Plan order of the tiles: tile i -> (b, g, t), as a plain launch maps
    workgroup i (sequences longest first by (P + C) * C, stable; with
    B * H_kv a multiple of 8, tile i's pseudo-request on XCD i % 8)."""
    n_t = _n_t(w)
    order = sorted(range(w.B), key=lambda b: -(w.prior[b] + w.chunk[b]) * w.chunk[b])
    xcd = (w.B * w.H_kv) % 8 == 0
    out = []
    for i in range(w.B * w.H_kv * n_t):
        if xcd:
            x, k = i & 7, i >> 3
            jj = k // n_t
            u, t = x + 8 * jj, k - jj * n_t
        else:
            u, t = i // n_t, i % n_t
        out.append((order[u // w.H_kv], u % w.H_kv, t))
    return out


def _model_cuts(w, T, lens, slots):
    """The plan's cut tiles, pieces per tile (plan order) and jobs per slot,
    from its description: work
    w_i = table entries up to the last block tile i's rows may see (at least
    1); A = max(ceil(sum / slots), 32), or the longest walk when that is
    within 2 job costs (12 units each) of it, and then nothing is cut; tile i
    runs whole when w_i - A < max(A / 8, 24), else its first A units on slot i
    and the rest as a tail; a slot's spare capacity is A - head - 12 (A growing
    by ceil(shortfall / slots with spare) until the tails fit, for at most 6
    rounds, then without the 12); the tails fill the spare capacity in order."""
    Th, lh = T.cpu().numpy(), lens.cpu().numpy()
    n_pb = (w.C_max + 31) // 32
    work = []
    for b, g, t in _plan_tiles(w):
        P, C = w.prior[b], w.chunk[b]
        if (t * 8) // w.G * 32 >= C:
            work.append(1)
            continue
        last_pb = min((t * 8 + 7) // w.G, n_pb - 1)
        kb_limit = (P + min(C, (last_pb + 1) * 32) - 1) // 64
        nkb = (P + C + 63) // 64
        n = min(max(int(lh[b, g]), 0), Th.shape[2])
        work.append(max(n - (nkb - 1 - kb_limit), 1))
    work = np.asarray(work, np.int64)
    n = len(work)
    assert n <= slots
    A = max(-(-int(work.sum()) // slots), BAL_MIN_SHARE)
    if int(work.max()) <= A + 2 * JOB_COST:
        return np.zeros(n, bool), np.ones(n, np.int64), np.array([1 if s < n else 0
                                                                  for s in range(slots)])
    heads = lambda: np.array([int(x) if x - A < max(A // 8, 2 * JOB_COST) else A for x in work])
    reserve = JOB_COST
    for rnd in range(7):
        if rnd == 6:
            reserve = 0
            break
        head = heads()
        spare = np.array([max(A - (int(head[s]) if s < n else 0) - reserve, 0) for s in range(slots)])
        dem, cap, nsp = int((work - head).sum()), int(spare.sum()), int((spare > 0).sum())
        if cap >= dem:
            break
        A += -(-(dem - cap) // max(nsp, 1))
    head = heads()
    tail = work - head
    tpre = np.concatenate([[0], np.cumsum(tail)])
    spare = np.array([max(A - (int(head[s]) if s < n else 0) - reserve, 0) for s in range(slots)])
    spre = np.concatenate([[0], np.cumsum(spare)])
    assert tpre[-1] <= spre[-1]
    # walk every slot's spare range and count the tiles whose tails it meets
    pieces = np.ones(n, np.int64)
    jobs = np.array([1 if s < n else 0 for s in range(slots)])
    for s in range(slots):
        lo, hi = int(spre[s]), min(int(spre[s + 1]), int(tpre[-1]))
        for i in range(n):
            if lo < hi and tail[i] > 0 and tpre[i] < hi and tpre[i + 1] > lo:
                pieces[i] += 1
                jobs[s] += 1
    assert jobs.max() <= 11
    return pieces > 1, pieces, jobs


def _check_cuts(ws, w, T, lens):
    """Pieces per tile read from the part numbering (a cut tile's parts; 0 for
    a tile run whole) equal the model's."""
    slots = min(torch.cuda.get_device_properties(0).multi_processor_count, PLAN_MAX_SLOTS)
    pre = _part_numbering(ws, w)
    got = np.diff(pre)
    want_cut, pieces, jobs = _model_cuts(w, T, lens, slots)
    want = np.where(want_cut, pieces, 0)
    assert pre[0] == 0 and np.array_equal(got, want), (np.nonzero(got != want)[0][:10], got[:16],
                                                       want[:16])
    return pieces, jobs


SHAPES = [
    # B, H_q, H_kv, D, prior, chunk, C_max, per-group densities, whether some slot runs a
    # third job (the jobs past the second run in a loop, compiled apart from the first two)
    (1, 8, 2, 128, [4096], [512], 512, [1.0, 0.05], False),
    (2, 16, 4, 128, [4096, 1024], [512, 256], 512, [1.0, 0.05, 0.3, 0.0], True),
    (3, 8, 1, 64, [1920, 0, 4096], [384, 256, 192], 448, [0.2], True),
    (2, 4, 4, 64, [6144, 640], [128, 64], 192, [0.5, 0.0, 1.0, 0.02], True),
]


@pytest.mark.parametrize("B,H_q,H_kv,D,prior,chunk,C_max,dens,third_job", SHAPES)
def test_balanced_small_full_parity(B, H_q, H_kv, D, prior, chunk, C_max, dens, third_job):
    w = gen.make_custom(B, H_q, H_kv, D, prior, chunk, "bf16", 300 + sum(prior) % 97,
                        _by_group(dens, H_q // H_kv), C_max=C_max, name="balanced_small")
    say(f"balanced small B={B} H={H_q}/{H_kv} D={D} prior={prior} chunk={chunk} dens={dens}")
    d = Dev(w)
    T, lens = d.tables()
    ws = _workspace(w)
    O, lse = _balanced(d, T, lens, ws)
    torch.cuda.synchronize()
    pieces, jobs = _check_cuts(ws, w, T, lens)
    say(f"  tiles {pieces.size}, pieces {int(pieces.sum())}, cut tiles {int((pieces > 1).sum())}, "
        f"jobs per slot up to {int(jobs.max())}")
    assert (pieces > 1).any()  # small grids: tiles are cut to fill the compute units
    assert (jobs.max() >= 3) == third_job
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
    ws = _workspace(w)
    Ob, lb = _balanced(d, T, lens, ws)
    Op, lp = d.attention(T, lens, return_lse=True)
    torch.cuda.synchronize()
    pieces, _ = _check_cuts(ws, w, T, lens)
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
    ws = _workspace(w)
    O, lse = _balanced(d, T, lens, ws)
    torch.cuda.synchronize()
    pieces, _ = _check_cuts(ws, w, T, lens)
    say(f"  pieces per tile {sorted(set(pieces.tolist()))}")
    assert pieces.min() > 1
    rows = sample_rows(w, seed=zlib.crc32(variant.encode()) % 1000, heads_per_group=4, extra=16)
    Or, lr = oracle_rows(w, rows)
    r = torch.from_numpy(rows).cuda()
    compare_bf16(to_np(O[r[:, 0], r[:, 1], r[:, 2]]), Or, f"{len(rows)} sampled rows")
    check_lse(to_np(lse[r[:, 0], r[:, 1], r[:, 2]]), lr)
    assert bool(torch.isfinite(O).all())


def test_balanced_groupshared_128k_sampled():
    # the 128K chunk with one mask per KV group: group tables of 119-172 blocks, so the
    # longest groups' tiles are cut and slots run up to four jobs (the loop past the first
    # two included); the part numbering matches the model, sampled rows match the oracle
    w = gen.make_workload("llama8b_128k", variant="groupshared")
    say("balanced groupshared 128K")
    d = Dev(w)
    T, lens = d.tables()
    ws = _workspace(w)
    O, lse = _balanced(d, T, lens, ws)
    torch.cuda.synchronize()
    pieces, jobs = _check_cuts(ws, w, T, lens)
    say(f"  cut tiles {int((pieces > 1).sum())}, jobs per slot up to {int(jobs.max())}")
    assert (pieces > 1).any() and jobs.max() >= 3
    rows = sample_rows(w, seed=101, heads_per_group=4, extra=8)
    Or, lr = oracle_rows(w, rows)
    r = torch.from_numpy(rows).cuda()
    compare_bf16(to_np(O[r[:, 0], r[:, 1], r[:, 2]]), Or, f"{len(rows)} sampled rows")
    check_lse(to_np(lse[r[:, 0], r[:, 1], r[:, 2]]), lr)


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


def test_balanced_more_tiles_than_slots_runs_plain_kernel():
    # 8 sequences x 8 groups x 16 tiles = 1024 tiles, more than the compute
    # units: the call runs the plain kernel (bit for bit) and leaves the
    # workspace alone
    B, H_q, H_kv, D, C_max = 8, 32, 8, 128, 1024
    rng = np.random.default_rng(95)
    prior = [64 * int(x) for x in rng.integers(0, 64, B)]
    chunk = [64 * int(x) for x in rng.integers(1, 17, B)]
    chunk[0] = C_max
    w = gen.make_custom(B, H_q, H_kv, D, prior, chunk, "bf16", 96,
                        _by_group([1.0, 0.1, 0.5, 0.0, 0.3, 1.0, 0.05, 0.7], H_q // H_kv),
                        C_max=C_max, name="balanced_more_tiles")
    n = B * H_kv * _n_t(w)
    if n <= min(torch.cuda.get_device_properties(0).multi_processor_count, PLAN_MAX_SLOTS):
        pytest.skip("needs more tiles than compute units")
    say(f"balanced with {n} tiles")
    d = Dev(w)
    T, lens = d.tables()
    ws = _workspace(w)
    O, lse = _balanced(d, T, lens, ws)
    Op, lp = d.attention(T, lens, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(O, Op) and torch.equal(lse, lp)
    assert not ws.any()
    rows = sample_rows(w, seed=97, heads_per_group=1, extra=4)
    Or, lr = oracle_rows(w, rows)
    r = torch.from_numpy(rows).cuda()
    compare_bf16(to_np(O[r[:, 0], r[:, 1], r[:, 2]]), Or, f"{len(rows)} sampled rows")
    check_lse(to_np(lse[r[:, 0], r[:, 1], r[:, 2]]), lr)


def test_balanced_garbage_workspace_and_graph_replay():
    # a workspace of garbage bytes, then one captured call replayed three times
    # with eager calls on the same workspace between the replays: every result
    # equals the first eager one bit for bit
    w = gen.make_custom(1, 16, 4, 128, [8192], [1024], "bf16", 98,
                        _by_group([1.0, 0.05, 0.4, 0.1], 4), name="balanced_graph")
    say("balanced: garbage workspace, graph replays between eager calls")
    d = Dev(w)
    T, lens = d.tables()
    n = ca.balanced_workspace_size(w.B, w.H_q, w.H_kv, w.C_max, w.D)
    ws = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    O_ref, l_ref = _balanced(d, T, lens, ws)
    O_ref, l_ref = O_ref.clone(), l_ref.clone()
    torch.cuda.synchronize()
    Or, lr = oracle_full(w)
    compare_bf16(to_np(O_ref), Or, "O")
    live = np.isfinite(lr)
    check_lse(to_np(l_ref)[live], lr[live])
    O_g = torch.empty_like(d.q)
    l_g = torch.empty((w.B, w.H_q, w.C_max), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up call outside the capture
        ca.chunk_attention(d.q, d.k, d.v, T, lens, w.prior, w.chunk, w.scale, out=O_g,
                           lse=l_g, balanced=True, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ca.chunk_attention(d.q, d.k, d.v, T, lens, w.prior, w.chunk, w.scale, out=O_g,
                           lse=l_g, balanced=True, workspace=ws)
    for rep in range(3):
        O_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(O_g, O_ref) and torch.equal(l_g, l_ref), f"replay {rep}"
        O_e, l_e = _balanced(d, T, lens, ws)  # eager call in between
        torch.cuda.synchronize()
        assert torch.equal(O_e, O_ref) and torch.equal(l_e, l_ref), f"eager {rep}"


def test_balanced_past_workspace_limit_runs_plain_kernel():
    # more tiles (B * H_kv * tiles per group = 17 * 8 * 64) than the workspace
    # is ever sized for (1024): 16 bytes of workspace, the plain kernel runs
    # (same result, bit for bit)
    B, H_q, H_kv, D, C_max = 17, 64, 8, 64, 2048
    rng = np.random.default_rng(91)
    prior = [64 * int(x) for x in rng.integers(0, 12, B)]
    chunk = [64 * int(x) for x in rng.integers(1, 33, B)]
    chunk[0] = C_max
    w = gen.make_custom(B, H_q, H_kv, D, prior, chunk, "bf16", 92,
                        _by_group([1.0, 0.1, 0.5, 0.0, 0.3, 1.0, 0.05, 0.7], H_q // H_kv),
                        C_max=C_max, name="balanced_many_tiles")
    assert B * H_kv * _n_t(w) > PLAN_MAX_SLOTS
    assert ca.balanced_workspace_size(B, H_q, H_kv, C_max, D) == 16
    say(f"balanced with {B * H_kv * _n_t(w)} tiles")
    d = Dev(w)
    T, lens = d.tables()
    ws = _workspace(w)
    O, lse = _balanced(d, T, lens, ws)
    Op, lp = d.attention(T, lens, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(O, Op) and torch.equal(lse, lp)
    rows = sample_rows(w, seed=93, heads_per_group=1, extra=2)
    Or, lr = oracle_rows(w, rows)
    r = torch.from_numpy(rows).cuda()
    compare_bf16(to_np(O[r[:, 0], r[:, 1], r[:, 2]]), Or, f"{len(rows)} sampled rows")
    check_lse(to_np(lse[r[:, 0], r[:, 1], r[:, 2]]), lr)
    for b in range(B):
        assert bool((O[b, :, chunk[b]:] == 0).all())
