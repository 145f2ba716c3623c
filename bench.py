#!/usr/bin/env python3
"""Benchmark of the CompactAttention chunked-prefill hot path on one MI355X.

One step = the whole path on one synthetic batch: Block-Union table build
(ca_build_union_tables) + zero-copy chunk attention (ca_chunk_attention), on
the 128K-context LLaMA-3.1-8B-shaped chunk: B=1, 32 query / 8 KV heads, D=128,
129024 cached tokens + a 2048-token chunk, bf16, per-head mask = sink + last 8
prior blocks + Bernoulli(0.05) per (head, Q-block, KV-block) cell.  The dense
baseline (all-ones mask, the same kernel fed every block) and a column-shared
mask variant (one draw per (head, KV-block)) and a group-shared one (one draw
per (KV group, KV-block): every mask row of a group is the group's union) are
timed beside it, and so is
the explicit-compaction baseline (ca_compact_kv gathers the selected blocks,
then the same kernel runs on the compact buffer), and the block-sparse-kernel
baseline (ca_chunk_attention_rows: each Q-block of each head attends its own
mask row, no union).

    python bench.py [--steps K] [--warmup W] [--gpus 1]

prints ONE JSON line.  ``value`` is the effective TFLOP/s of a whole step
(algorithmic FLOPs: 4*D per admissible query/key pair over the selected
blocks, causal triangle included).  Inputs are resident in HBM before timing.

Profiling helpers (for rocprofv3 runs): ``--profile attn|union|compact|prefill|copy`` runs only
that kernel a few times (``copy`` = a plain device copy of known size, used to
scale the HBM byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E (published)
PEAK_CLOCK_GHZ = 2.4       # the engine clock the published matrix peak assumes
WORKLOAD = "llama8b_128k"
PMC_SUMMARY = os.path.join(ROOT, "profiles", "chunk_attn_bf16_llama8b_128k_pmc.txt")
KERNEL_SRC = os.path.join(ROOT, "chunked_prefill_sparse_amd", "csrc", "chunk_attn_bf16.hip")
KERNEL_HDR = os.path.join(ROOT, "chunked_prefill_sparse_amd", "csrc", "attn_bf16_common.hpp")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- work accounting


def admissible_pairs(T: np.ndarray, lens: np.ndarray, prior, chunk, G: int) -> int:
    """Number of (query, key) pairs the path must compute: for every query head
    and chunk row i, the keys t <= prior+i of the blocks in T[b,g]."""
    total = 0
    for b in range(T.shape[0]):
        P, C = int(prior[b]), int(chunk[b])
        i = np.arange(C, dtype=np.int64)
        for g in range(T.shape[1]):
            blocks = T[b, g, :lens[b, g]].astype(np.int64)
            start = blocks * 64
            full = blocks[start + 63 <= P]  # prior blocks below every row: 64 keys each
            pairs = full.size * 64 * C
            part = start[start + 63 > P]
            if part.size:
                # keys start..start+63 (and < P+C) with t <= P+i
                cnt = np.clip(P + i[None, :] - part[:, None] + 1, 0, 64)
                cnt = np.minimum(cnt, np.clip(P + C - part[:, None], 0, 64))
                pairs += int(cnt.sum())
            total += pairs * G
    return int(total)


def admissible_pairs_rows(mask: np.ndarray, prior, chunk) -> int:
    """(query, key) pairs of block-sparse execution: Q-block qb of each head
    attends the blocks of its own mask row; 64*64 pairs per block wholly below
    the Q-block, the causal triangle (2080 pairs) on its diagonal block."""
    total = 0
    for b in range(mask.shape[0]):
        P, C = int(prior[b]), int(chunk[b])
        nq, pblk = C // 64, P // 64
        m = mask[b, :, :nq, :pblk + nq] != 0
        below = np.tril(np.ones((nq, nq), bool), -1)  # chunk blocks wholly below each Q-block
        full = m[:, :, :pblk].sum() + (m[:, :, pblk:] & below[None]).sum()
        diag = m[:, np.arange(nq), pblk + np.arange(nq)].sum()
        total += int(full) * 64 * 64 + int(diag) * 2080
    return total


def algorithmic(w, T, lens):
    pairs = admissible_pairs(T, lens, w.prior, w.chunk, w.G)
    flops = 4 * w.D * pairs
    esz = 2 if w.dtype == "bf16" else 4
    kv = 2 * 64 * int(lens.sum()) * w.D * esz
    qo = 2 * w.B * w.H_q * w.C_max * w.D * esz
    meta = T.size * 4 + lens.size * 4
    return flops, kv + qo + meta, pairs


# --------------------------------------------------------------------------- timing


def time_calls(fn, reps, stream):
    """Per-call durations (ms) from HIP events recorded on the launch stream."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def time_calls_cold(fn, reps, stream, scratch):
    """Like time_calls, but a write over ``scratch`` (>= 512 MiB, larger than the
    caches) runs before each call, outside the timed events, so every call
    starts with cold L2 and MALL."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        scratch.fill_(1)
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def pct(xs, q):
    return float(np.percentile(np.asarray(xs), q))


# --------------------------------------------------------------------------- cpu baseline


def cpu_baseline(w, seconds_budget=20.0):
    """The oracle as it stands, on a bounded sample of the same workload: the
    union of the whole mask, then attention for every chunk row of the query
    heads of one KV group after another until the time budget is spent, timed
    on this host's cores."""
    import gen
    from oracle import chunk_attention_rows_ref, union_tables_ref
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([int(i.get("num_threads", 1)) for i in info] or [1])
        blas = ",".join(sorted({str(i.get("internal_api", "?")) for i in info
                                if i.get("user_api") == "blas"})) or "unknown"
    except Exception:
        threads, blas = 1, "unknown"
    t0 = time.perf_counter()
    T, ln = union_tables_ref(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
    t_union = time.perf_counter() - t0
    q, k, v = (gen.tensor_to_f32(x) for x in (w.q, w.k, w.v))
    C, P = w.chunk[0], w.prior[0]
    elapsed, flops, groups, rows_done = 0.0, 0, 0, 0
    for g in range(w.H_kv):
        if elapsed >= seconds_budget:
            break
        rows = np.array([(0, h, i) for h in range(g * w.G, (g + 1) * w.G) for i in range(C)],
                        np.int64)
        t0 = time.perf_counter()
        chunk_attention_rows_ref(q, k, v, T, ln, w.prior, w.chunk, w.scale, rows)
        elapsed += time.perf_counter() - t0
        flops += 4 * w.D * admissible_pairs(T[:, g:g + 1], ln[:, g:g + 1], w.prior, w.chunk, w.G)
        groups += 1
        rows_done += rows.shape[0]
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle on {WORKLOAD}: union tables of the whole mask "
                   f"({t_union:.2f} s), then attention for all {C} chunk rows of the {w.G} "
                   f"query heads of {groups} of {w.H_kv} KV groups ({rows_done} rows) in "
                   f"{elapsed:.1f} s; value = algorithmic FLOPs of those rows / their time"),
        "host_cpus": os.cpu_count(),
        "blas": blas,
        "note": "NumPy element-wise work (exp, max) runs on one thread; the products use BLAS threads",
        "cpu_model": platform.processor() or platform.machine(),
    }


# --------------------------------------------------------------------------- every config


def dense_tables(w, dev):
    """The all-blocks table of a workload (every block of each sequence, the
    dense baseline the same kernel runs) and its lengths."""
    import torch
    T = torch.full((w.B, w.H_kv, w.NKB_max), -1, dtype=torch.int32)
    ln = torch.zeros((w.B, w.H_kv), dtype=torch.int32)
    for b, n in enumerate(w.n_kv_blocks):
        T[b, :, :n] = torch.arange(n, dtype=torch.int32)
        ln[b] = n
    return T.to(dev), ln.to(dev)


def union_kernel_us(fn, calls=50):
    """Kernel time of one union call: ``calls`` calls recorded into a HIP graph,
    replayed, and timed with HIP events (no per-call host launch work)."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = []
    for _ in range(5):
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        reps.append(a.elapsed_time(b) * 1e3 / calls)
    del g
    return statistics.median(reps)


def blocks_summary(w, lh):
    """[sum of len, mean len per (sequence, KV group), mean per-head Q-block
    union, mean blocks per sequence] (+ the achieved density of the prior cells
    for vertical-slash masks)."""
    per_head = []
    for b in range(w.B):
        nq, nkb = w.n_q_blocks[b], w.n_kv_blocks[b]
        per_head.append(w.mask[b, :, :nq, :nkb].any(axis=1).sum(axis=-1).mean())
    all_blocks = float(np.mean([n for n in w.n_kv_blocks]))
    r = [int(lh.sum()), round(float(lh.mean()), 1), round(float(np.mean(per_head)), 1),
         round(all_blocks, 1)]
    if w.meta.get("mask") == "vertical_slash":
        pb = w.prior[0] // 64
        r.append(round(float(w.mask[:, :, :w.n_q_blocks[0], :pb].mean()), 4))
    return r


def measure_config(w, dev, stream, reps, q=None, k=None, v=None, dense_ms=None):
    """One workload on the GPU: union tables (per call and kernel only), chunk
    attention (median, p10, p90 of ``reps`` HIP-event-timed calls), the same
    kernel over every block (x vs dense), and the work accounting."""
    import torch
    import chunked_prefill_sparse_amd as ca
    q = w.q.to(dev) if q is None else q
    k = w.k.to(dev) if k is None else k
    v = w.v.to(dev) if v is None else v
    mask = torch.from_numpy(w.mask).to(dev)
    T = torch.empty((w.B, w.H_kv, w.NKB_max), dtype=torch.int32, device=dev)
    lens = torch.empty((w.B, w.H_kv), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)

    def tables():
        ca.build_union_tables(mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks, T=T, lens=lens)

    def attn(T_=T, l_=lens, **kw):
        ca.chunk_attention(q, k, v, T_, l_, w.prior, w.chunk, w.scale, out=out, **kw)

    tables()
    torch.cuda.synchronize()
    Th, lh = T.cpu().numpy(), lens.cpu().numpy()
    flops, bytes_alg, pairs = algorithmic(w, Th, lh)
    attn()
    a_ms = time_calls(attn, reps, stream)
    u_ms = time_calls(tables, reps, stream)
    u_kernel = union_kernel_us(tables)
    med = statistics.median(a_ms)
    eff = flops / (med * 1e-3) / 1e12
    r = dict(
        ms=[round(med, 4), round(pct(a_ms, 10), 4), round(pct(a_ms, 90), 4)],
        union_us=[round(statistics.median(u_ms) * 1e3, 2), round(u_kernel, 2)],
        tflops=round(eff, 2),
        hbm_GBps=round(bytes_alg / (med * 1e-3) / 1e9, 1),
        len=blocks_summary(w, lh),
    )
    if w.dtype == "bf16":
        r["mfma"] = round(eff / PEAK_BF16_TFLOPS, 4)
    else:  # fp32 on the vector ALUs: latency-bound, also run split 8 ways
        ws = torch.empty(ca.workspace_size(w.B, w.H_q, w.C_max, w.D, 8), dtype=torch.uint8,
                         device=dev)
        attn(n_splits=8, workspace=ws)
        s_ms = statistics.median(time_calls(lambda: attn(n_splits=8, workspace=ws), reps, stream))
        r["split8_ms"] = round(s_ms, 4)
        r["split8_tflops"] = round(flops / (s_ms * 1e-3) / 1e12, 3)
    if dense_ms is None:
        Td, ld = dense_tables(w, dev)
        attn(Td, ld)
        dense_ms = statistics.median(time_calls(lambda: attn(Td, ld), reps, stream))
    r["dense_ms"] = round(dense_ms, 4)
    r["x_dense"] = round(dense_ms / med, 3)
    return r


def oracle_seconds(w, arrays, full, runs=1):
    """The oracle on this workload, timed on the host cores: the whole output
    (``full``), else the slice of KV group 0 of every sequence, scaled to the
    whole workload by its share of the admissible pairs."""
    from oracle import chunk_attention_ref, union_tables_ref
    q, k, v = arrays
    t0 = time.perf_counter()
    Tr, lr = union_tables_ref(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
    t_union = time.perf_counter() - t0
    if full:
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            chunk_attention_ref(q, k, v, Tr, lr, w.prior, w.chunk, w.scale)
            ts.append(time.perf_counter() - t0)
        return dict(s=round(statistics.median(ts) + t_union, 3), runs=runs, sample="whole")
    G = w.G
    t0 = time.perf_counter()
    for b in range(w.B):
        chunk_attention_ref(q[b:b + 1, :G], k[b:b + 1, :1], v[b:b + 1, :1], Tr[b:b + 1, :1],
                            lr[b:b + 1, :1], w.prior[b:b + 1], w.chunk[b:b + 1], w.scale)
    t_slice = time.perf_counter() - t0
    part = admissible_pairs(Tr[:, :1], lr[:, :1], w.prior, w.chunk, G)
    whole = admissible_pairs(Tr, lr, w.prior, w.chunk, G)
    return dict(s=round(t_union + t_slice * whole / max(part, 1), 3),
                measured_s=round(t_union + t_slice, 3),
                sample=f"group 0 of each sequence ({part / whole:.3f} of the pairs), scaled")


def configs_leg(stream, reps, base, base_dev, results, oracle_budget):
    """Every synthetic config at one GPU: config 1 (fp32), config 2 (32K),
    config 3 (128K: pairwise, colshared, groupshared, dense), config 4 (ragged
    B=4) and the 12 points of config 5 (vertical-slash density sweep x heads
    identical / independent), each with the oracle's time on the host cores
    (whole output for configs 1 and 2, one KV group scaled for the rest, while
    ``oracle_budget`` seconds last)."""
    import torch
    import gen
    dev = base_dev[0].device
    cores = len(os.sched_getaffinity(0))
    out = {}
    spent = [0.0]

    def oracle(w, arrays, full, runs=1):
        if spent[0] >= oracle_budget:
            return dict(s=None, sample="skipped: oracle time budget spent")
        t0 = time.perf_counter()
        r = oracle_seconds(w, arrays, full, runs)
        spent[0] += time.perf_counter() - t0
        r["cores"] = cores
        return r

    def small(name, cfg, runs):
        w = gen.make_workload(name)
        r = measure_config(w, dev, stream, reps)
        r = dict(cfg=cfg, dtype=w.dtype, **r)
        r["oracle"] = oracle(w, tuple(gen.tensor_to_f32(x) for x in (w.q, w.k, w.v)), True, runs)
        log(f"config {cfg} {name}: attention {r['ms'][0]:.4f} ms ({r['tflops']:.1f} TFLOP/s), "
            f"union {r['union_us'][0]:.1f} us (kernel {r['union_us'][1]:.1f}), "
            f"x{r['x_dense']:.2f} vs dense, oracle {r['oracle']['s']} s")
        return r

    out["tiny_f32"] = small("tiny_f32", 1, 5)
    out["llama8b_32k"] = small("llama8b_32k", 2, 1)
    torch.cuda.empty_cache()

    q, k, v = base_dev
    base_arrays = tuple(gen.tensor_to_f32(x) for x in (base.q, base.k, base.v))
    dense_ms = results["dense"]["attn_ms_median"]
    for variant in ("pairwise", "colshared", "groupshared", "dense"):
        w = gen.make_workload("llama8b_128k", variant=variant, with_tensors=False)
        r = measure_config(w, dev, stream, reps, q, k, v, dense_ms=dense_ms)
        r = dict(cfg=3, dtype="bf16", **r)
        r["oracle"] = oracle(w, base_arrays, False)
        out[f"llama8b_128k.{variant}"] = r
        log(f"config 3 {variant}: attention {r['ms'][0]:.3f} ms ({r['tflops']:.0f} TFLOP/s), "
            f"union kernel {r['union_us'][1]:.1f} us, x{r['x_dense']:.2f} vs dense")
    for dn in gen.VSLASH_DENSITIES:
        for hm in gen.VSLASH_HEAD_MODES:
            w = gen.make_workload("vslash_128k", density=dn, heads=hm, with_tensors=False)
            r = measure_config(w, dev, stream, reps, q, k, v, dense_ms=dense_ms)
            r = dict(cfg=5, dtype="bf16", **r)
            r["oracle"] = oracle(w, base_arrays, False)
            out[f"vslash_128k.d{dn}.{hm}"] = r
            log(f"config 5 d={dn} {hm}: attention {r['ms'][0]:.3f} ms ({r['tflops']:.0f} "
                f"TFLOP/s), mean len {r['len'][1]} vs per-head {r['len'][2]}, "
                f"x{r['x_dense']:.2f} vs dense")
    del base_arrays
    w = gen.make_workload("ragged_b4")
    r = measure_config(w, dev, stream, reps)
    r = dict(cfg=4, dtype="bf16", **r)
    r["oracle"] = oracle(w, tuple(gen.tensor_to_f32(x) for x in (w.q, w.k, w.v)), False)
    out["ragged_b4"] = r
    log(f"config 4 ragged_b4: attention {r['ms'][0]:.3f} ms ({r['tflops']:.0f} TFLOP/s), "
        f"x{r['x_dense']:.2f} vs dense")
    del w
    torch.cuda.empty_cache()
    return out


def markdown_table(line):
    """The benchmark's per-config table from a bench JSON line (``--table``)."""
    rows = ["| config / mask | attention ms (median; p10–p90) | union µs (per call; kernel) "
            "| eff. TFLOP/s | MFMA frac | alg. HBM GB/s | × vs dense "
            "| mean len / per-head Q-union / all blocks | oracle s (cores) |",
            "|---|---|---|---|---|---|---|---|---|"]
    for key, r in line["configs"].items():
        name, _, rest = key.partition(".")
        label = f"{r['cfg']} {name}" + (f" {rest}" if rest else "") + \
            (" (fp32)" if r["dtype"] == "f32" else "")
        m, u, ln = r["ms"], r["union_us"], r["len"]
        att = f"{m[0]:.3f}; {m[1]:.3f}–{m[2]:.3f}"
        if "split8_ms" in r:
            att += f" (8 splits: {r['split8_ms']:.3f})"
        o = r.get("oracle") or {}
        osec = "—" if o.get("s") is None else (
            f"{o['s']:.3g} ({o['cores']})" + ("" if o.get("sample") == "whole" else " est."))
        mf = f"{r['mfma']:.3f}" if "mfma" in r else "—"
        rows.append(f"| {label} | {att} | {u[0]:.1f}; {u[1]:.1f} | {r['tflops']:.1f} | {mf} "
                    f"| {r['hbm_GBps']:.0f} | {r['x_dense']:.2f} "
                    f"| {ln[1]:.0f} / {ln[2]:.0f} / {ln[3]:.0f} | {osec} |")
    return "\n".join(rows)


def _bench_line(rec):
    """The bench JSON line inside a record: the line itself, or a driver record
    holding it in its stdout tail."""
    if "configs" in rec:
        return rec
    for text in (rec.get("run", {}).get("stdout_tail", ""), rec.get("tail", "")):
        for ln in text.splitlines():
            if ln.startswith("{") and '"configs"' in ln:
                return json.loads(ln)
    raise SystemExit("no bench line with a configs object in that record")


# --------------------------------------------------------------------------- one GPU's TP share


def tp_shard_leg(stream, reps):
    """One GPU's share of the 128K chunk under tensor parallelism over KV heads:
    4 query heads and their one KV head (only 64 workgroups of 128 rows), with
    and without split-KV (each table cut into n ranges, then merged)."""
    import torch
    import gen
    import chunked_prefill_sparse_amd as ca
    from gen.workloads import _bernoulli_sink_local
    out = {}
    for variant in ("pairwise", "colshared"):
        cs = variant == "colshared"
        w = gen.make_custom(1, 4, 1, 128, [129024], [2048], "bf16", 1008,
                            lambda rng, b, H, nq, pb: _bernoulli_sink_local(
                                rng, H, nq, pb, 0.05, 8, colshared=cs),
                            name=f"tp_shard_128k_{variant}")
        q, k, v = w.q.cuda(), w.k.cuda(), w.v.cuda()
        mask = torch.from_numpy(w.mask).cuda()
        T, lens = ca.build_union_tables(mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
        o = torch.empty_like(q)
        torch.cuda.synchronize()
        flops = 4 * w.D * admissible_pairs(T.cpu().numpy(), lens.cpu().numpy(), w.prior, w.chunk,
                                           w.G)
        res = {}
        for n in (1, 2, 4, 8):
            ws = torch.empty(max(ca.workspace_size(1, 4, 2048, 128, n), 16), dtype=torch.uint8,
                             device=q.device)
            fn = lambda: ca.chunk_attention(q, k, v, T, lens, w.prior, w.chunk, w.scale, out=o,  # noqa: E731
                                            n_splits=n, workspace=ws)
            fn()
            ms = statistics.median(time_calls(fn, reps, stream))
            res[n] = ms
        best = min(res, key=res.get)
        bws = torch.empty(ca.balanced_workspace_size(1, 4, 1, 2048, 128), dtype=torch.uint8,
                          device=q.device)
        fb = lambda: ca.chunk_attention(q, k, v, T, lens, w.prior, w.chunk, w.scale, out=o,  # noqa: E731
                                        balanced=True, workspace=bws)
        fb()
        bal = statistics.median(time_calls(fb, reps, stream))
        out[variant] = dict(
            ms_by_splits={str(n_): round(t_, 4) for n_, t_ in res.items()},
            eff_tflops_no_split=round(flops / (res[1] * 1e-3) / 1e12, 1),
            best_splits=best, eff_tflops_best=round(flops / (res[best] * 1e-3) / 1e12, 1),
            balanced_ms=round(bal, 4), eff_tflops_balanced=round(flops / (bal * 1e-3) / 1e12, 1))
        log(f"tp_shard_128k {variant}: no split {res[1]:.3f} ms "
            f"({out[variant]['eff_tflops_no_split']:.0f} TFLOP/s), best n={best} "
            f"{res[best]:.3f} ms ({out[variant]['eff_tflops_best']:.0f} TFLOP/s), balanced "
            f"{bal:.3f} ms ({out[variant]['eff_tflops_balanced']:.0f} TFLOP/s)")
        del q, k, v, mask, T, lens, o
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- whole prefill


def prefill_leg(stream, budget=32, local=8, overlap=True):
    """A 128K prompt in 64 chunks of 2048 (planted-structure synthetic stream):
    per chunk, append its keys and values to the cache, pool the new key
    blocks and the queries, make the top-k block mask, build the union tables
    and run zero-copy attention (also timed with balanced attention, for
    reference); the dense baseline appends and runs the same attention over
    every block.  The caches start empty.  Cumulative times from HIP events on
    the launch stream, for the Python loop of calls and for the same calls
    recorded into HIP graphs and replayed; with overlap, also for the run that
    issues each chunk's append and selection on a second stream ahead of the
    attention (left out of kernel traces, whose per-kernel durations assume
    kernels that do not run side by side)."""
    import torch
    import gen
    from chunked_prefill_sparse_amd.prefill import ChunkedPrefill
    log("generating prefill_128k stream ...")
    s = gen.make_prefill_stream("prefill_128k")
    k_src, v_src = s.k.cuda(), s.v.cuda()
    kv = [(k_src[:, :, c * s.C:(c + 1) * s.C].contiguous(),
           v_src[:, :, c * s.C:(c + 1) * s.C].contiguous()) for c in range(s.n_chunks)]
    del k_src, v_src
    k = torch.zeros((1, s.H_kv, s.L, s.D), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    qs = [s.q_chunk(c).cuda() for c in range(s.n_chunks)]
    drv = ChunkedPrefill(k, v, s.H_q, s.C, budget=budget, local=local, balanced=False)
    drv_bal = ChunkedPrefill(k, v, s.H_q, s.C, budget=budget, local=local, balanced=True)
    dense_lens = [drv.dense_lens(c * s.C) for c in range(s.n_chunks)]
    priors = [c * s.C for c in range(s.n_chunks)]
    torch.cuda.synchronize()
    # untimed pass: work accounting per chunk
    flops = flops_dense = 0
    frac = []
    for c in range(s.n_chunks):
        P = c * s.C
        drv.step(qs[c], P, k_chunk=kv[c][0], v_chunk=kv[c][1])
        T, ln = drv.T.cpu().numpy(), drv.lens.cpu().numpy()
        flops += 4 * s.D * admissible_pairs(T, ln, [P], [s.C], s.G)
        nkb = (P + s.C) // 64
        Td = np.broadcast_to(np.arange(nkb, dtype=np.int32), (1, s.H_kv, nkb))
        flops_dense += 4 * s.D * admissible_pairs(Td, np.full((1, s.H_kv), nkb), [P], [s.C], s.G)
        frac.append(float(ln.sum()) / (s.H_kv * nkb))

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def run_sparse():
        for c in range(s.n_chunks):
            drv.step(qs[c], priors[c], k_chunk=kv[c][0], v_chunk=kv[c][1])

    def run_append():
        for c in range(s.n_chunks):
            drv.append(kv[c][0], kv[c][1], priors[c])

    def run_select():
        for c in range(s.n_chunks):
            drv.select(qs[c], priors[c])

    def run_append_select():  # the fused call the sparse step issues
        for c in range(s.n_chunks):
            drv.append_select(kv[c][0], kv[c][1], qs[c], priors[c])

    def run_select_separate():  # the same selection through the six separate launches
        for c in range(s.n_chunks):
            drv.select_separate(qs[c], priors[c])

    def run_dense():
        for c in range(s.n_chunks):
            drv.step_dense(qs[c], priors[c], dense_lens[c], k_chunk=kv[c][0], v_chunk=kv[c][1])

    def run_balanced():  # the same loop with balanced attention, for reference
        for c in range(s.n_chunks):
            drv_bal.step(qs[c], priors[c], k_chunk=kv[c][0], v_chunk=kv[c][1])

    # one graph of a whole chunk step, captured once and replayed for every chunk:
    # each chunk's inputs are copied into the graph's buffers first
    drv_dl = ChunkedPrefill(k, v, s.H_q, s.C, budget=budget, local=local)
    q_buf, k_buf, v_buf = torch.empty_like(qs[0]), torch.empty_like(kv[0][0]), \
        torch.empty_like(kv[0][1])

    def load_chunk(c):
        q_buf.copy_(qs[c])
        k_buf.copy_(kv[c][0])
        v_buf.copy_(kv[c][1])
        drv_dl.set_prior(priors[c])

    def run_loads():
        for c in range(s.n_chunks):
            load_chunk(c)

    def run_overlap():  # each chunk's append and selection on a second stream, ahead
        drv.run(qs, priors, kv_chunks=kv, overlap=True)

    def run_overlap_balanced():
        drv_bal.run(qs, priors, kv_chunks=kv, overlap=True)

    reps = 3
    run_sparse()
    run_dense()
    sparse_ms = statistics.median(timed(run_sparse) for _ in range(reps))
    append_ms = statistics.median(timed(run_append) for _ in range(reps))
    select_ms = statistics.median(timed(run_select) for _ in range(reps))
    select_sep_ms = statistics.median(timed(run_select_separate) for _ in range(reps))
    appsel_ms = statistics.median(timed(run_append_select) for _ in range(reps))
    dense_ms = statistics.median(timed(run_dense) for _ in range(reps))
    attn_ms = sparse_ms - appsel_ms
    run_balanced()
    bal_ms = statistics.median(timed(run_balanced) for _ in range(reps))
    if overlap:
        run_overlap()
        run_overlap_balanced()
        ov_ms = statistics.median(timed(run_overlap) for _ in range(reps))
        ovb_ms = statistics.median(timed(run_overlap_balanced) for _ in range(reps))
    # the same call sequences recorded once into HIP graphs and replayed: the
    # GPU time without the per-call host work of the loop above
    g_sparse = drv.capture(qs, priors, kv_chunks=kv)
    g_select = drv.capture(qs, priors, select_only=True)
    g_appsel = drv.capture(qs, priors, select_only=True, kv_chunks=kv)
    g_select_sep = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_select_sep):
        run_select_separate()
    g_dense = drv.capture(qs, priors, dense=True, kv_chunks=kv)
    g_bal = drv_bal.capture(qs, priors, kv_chunks=kv)
    g_ov = drv.capture(qs, priors, kv_chunks=kv, overlap=True) if overlap else None
    g_ovb = drv_bal.capture(qs, priors, kv_chunks=kv, overlap=True) if overlap else None
    load_chunk(0)
    drv_dl.step_devlen(q_buf, k_buf, v_buf)
    g_chunk = drv_dl.capture_chunk(q_buf, k_buf, v_buf)

    def run_chunk_graph():
        for c in range(s.n_chunks):
            load_chunk(c)
            g_chunk.replay()

    g_sparse.replay()
    g_dense.replay()
    g_bal.replay()
    run_chunk_graph()
    if overlap:
        g_ov.replay()
        g_ovb.replay()
    gs_ms = statistics.median(timed(g_sparse.replay) for _ in range(reps))
    gb_ms = statistics.median(timed(g_bal.replay) for _ in range(reps))
    gsel_ms = statistics.median(timed(g_select.replay) for _ in range(reps))
    gsel_sep_ms = statistics.median(timed(g_select_sep.replay) for _ in range(reps))
    gappsel_ms = statistics.median(timed(g_appsel.replay) for _ in range(reps))
    gd_ms = statistics.median(timed(g_dense.replay) for _ in range(reps))
    gchunk_ms = statistics.median(timed(run_chunk_graph) for _ in range(reps))
    loads_ms = statistics.median(timed(run_loads) for _ in range(reps))
    if overlap:
        gov_ms = statistics.median(timed(g_ov.replay) for _ in range(reps))
        govb_ms = statistics.median(timed(g_ovb.replay) for _ in range(reps))
    moved = 2 * 2 * s.n_chunks * s.H_kv * s.C * s.D * 2  # K and V, read once and written once
    r = dict(
        chunks=s.n_chunks, chunk=s.C, prompt=s.L, budget_blocks=budget, local_blocks=local,
        total_ms=round(sparse_ms, 3), append_select_ms=round(appsel_ms, 3),
        append_ms=round(append_ms, 3),
        append_GBps=round(moved / (append_ms * 1e-3) / 1e9, 1), select_ms=round(select_ms, 3),
        select_separate_ms=round(select_sep_ms, 3),
        attention_ms=round(attn_ms, 3), dense_total_ms=round(dense_ms, 3),
        x_vs_dense=round(dense_ms / sparse_ms, 3),
        attention_eff_tflops=round(flops / (attn_ms * 1e-3) / 1e12, 1),
        dense_eff_tflops=round(flops_dense / ((dense_ms - append_ms) * 1e-3) / 1e12, 1),
        work_frac_of_dense=round(flops / flops_dense, 4),
        union_block_frac_first_mid_last=[round(frac[0], 3), round(frac[len(frac) // 2], 3),
                                         round(frac[-1], 3)],
        balanced=dict(total_ms=round(bal_ms, 3),
                      attention_ms=round(bal_ms - appsel_ms, 3),
                      x_vs_dense=round(dense_ms / bal_ms, 3),
                      attention_eff_tflops=round(
                          flops / ((bal_ms - appsel_ms) * 1e-3) / 1e12, 1)),
        graph=dict(total_ms=round(gs_ms, 3), append_select_ms=round(gappsel_ms, 3),
                   select_ms=round(gsel_ms, 3),
                   select_separate_ms=round(gsel_sep_ms, 3),
                   dense_total_ms=round(gd_ms, 3), x_vs_dense=round(gd_ms / gs_ms, 3),
                   balanced_total_ms=round(gb_ms, 3),
                   balanced_x_vs_dense=round(gd_ms / gb_ms, 3),
                   # one graph of a chunk step (device chunk offset) replayed per chunk,
                   # with the copies of each chunk's Q, K, V into its input buffers
                   one_chunk_graph_total_ms=round(gchunk_ms, 3),
                   one_chunk_graph_input_copies_ms=round(loads_ms, 3)),
        # append + selection on a second stream, ahead of the attention
        overlap=dict(total_ms=round(ov_ms, 3), x_vs_dense=round(dense_ms / ov_ms, 3),
                     balanced_total_ms=round(ovb_ms, 3),
                     balanced_x_vs_dense=round(dense_ms / ovb_ms, 3),
                     graph_total_ms=round(gov_ms, 3), graph_x_vs_dense=round(gd_ms / gov_ms, 3),
                     graph_balanced_total_ms=round(govb_ms, 3),
                     graph_balanced_x_vs_dense=round(gd_ms / govb_ms, 3)) if overlap else None,
        data=("synthetic planted-structure stream: K, V, Q ~ N(0,1), 3% salient KV blocks per "
              "KV head shifted along a per-head direction that the group's queries share; the "
              "caches start empty and each chunk appends its own K/V"),
    )
    log(f"prefill_128k: total {sparse_ms:.2f} ms (append + select {appsel_ms:.2f}; alone: append "
        f"{append_ms:.2f}, select {select_ms:.2f}; attention {attn_ms:.2f}) vs dense "
        f"{dense_ms:.2f} ms -> x{dense_ms / sparse_ms:.2f}; "
        f"union fraction first/mid/last {r['union_block_frac_first_mid_last']}")
    log(f"prefill_128k with balanced attention: total {bal_ms:.2f} ms -> x{dense_ms / bal_ms:.2f}")
    log(f"prefill_128k as HIP graphs: total {gs_ms:.2f} ms (append + select {gappsel_ms:.2f}, "
        f"select {gsel_ms:.2f}, through the "
        f"separate calls {gsel_sep_ms:.2f}) vs dense {gd_ms:.2f} ms -> x{gd_ms / gs_ms:.2f}; "
        f"with balanced attention {gb_ms:.2f} ms -> x{gd_ms / gb_ms:.2f}")
    if overlap:
        log(f"prefill_128k overlapped (append + selection ahead, on a second stream): "
            f"{ov_ms:.2f} ms -> x{dense_ms / ov_ms:.2f}, balanced {ovb_ms:.2f} ms; as graphs "
            f"{gov_ms:.2f} ms -> x{gd_ms / gov_ms:.2f}, balanced {govb_ms:.2f} ms -> "
            f"x{gd_ms / govb_ms:.2f}")
    log(f"prefill_128k, one graph of a chunk step replayed per chunk: {gchunk_ms:.2f} ms, of "
        f"which copying each chunk's inputs into its buffers {loads_ms:.2f} ms")
    del qs, k, v, kv, drv, drv_bal, g_sparse, g_select, g_appsel, g_select_sep, g_dense, g_bal
    del g_ov, g_ovb, g_chunk, drv_dl, q_buf, k_buf, v_buf
    torch.cuda.empty_cache()
    return r


def select_profile_leg(calls, chunk=32, budget=32, local=8):
    """For counter runs of the fused append + selection: the 128K prefill stream
    appended and selected up to chunk `chunk` (prior 2048 * chunk), then
    `calls` more ca_append_select_chunk calls for that chunk, each printed with
    the algorithmic bytes of its four kernels (the counters of the last calls are
    the ones to read)."""
    import torch
    import gen
    from chunked_prefill_sparse_amd.prefill import ChunkedPrefill
    s = gen.make_prefill_stream("prefill_128k")
    k_src, v_src = s.k.cuda(), s.v.cuda()
    k = torch.zeros((1, s.H_kv, s.L, s.D), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    drv = ChunkedPrefill(k, v, s.H_q, s.C, budget=budget, local=local)

    def kv(c):
        return (k_src[:, :, c * s.C:(c + 1) * s.C].contiguous(),
                v_src[:, :, c * s.C:(c + 1) * s.C].contiguous())

    for c in range(chunk):
        kc, vc = kv(c)
        drv.append_select(kc, vc, s.q_chunk(c).cuda(), c * s.C)
    kc, vc = kv(chunk)
    q = s.q_chunk(chunk).cuda()
    torch.cuda.synchronize()
    P, C, D, Hq, Hkv = chunk * s.C, s.C, s.D, s.H_q, s.H_kv
    pblk, nq, nkb = P // 64, C // 64, s.L // 64
    nwords = (nkb + 31) // 32
    alg = {  # bytes each kernel must move at least (B = 1)
        "select_pool (with the append)": 2 * (2 * Hkv * C * D * 2) + Hq * C * D * 2
        + (Hkv + Hq) * nq * D * 4 + Hkv * 16 * nwords * 4,
        "block_scores": Hq * nq * D * 4 + Hkv * pblk * D * 4 + Hq * nq * pblk * 4,
        "topk_mask": Hq * nq * pblk * 4 + Hq * nq * nkb,
        "union_compact": Hkv * 16 * nwords * 4 + Hkv * nkb * 4 + Hkv * 4,
    }
    log(f"select profile: chunk {chunk}, prior {P}, algorithmic bytes per kernel {alg}")
    for i in range(calls):
        drv.append_select(kc, vc, q, P)
        torch.cuda.synchronize()
        log(f"append_select call {i}")


# --------------------------------------------------------------------------- main


_C_TOKEN = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/|\s+', re.S)


def code_hash(path):
    """First 16 hex digits of the SHA-256 of a C++/HIP source with its comments
    dropped and every run of white space folded to one blank, so that an edit
    to comments alone leaves it unchanged while any change to the code moves it."""
    def tok(m):
        t = m.group(0)
        if t.startswith("//") or t.startswith("/*") or t.isspace():
            return " "
        return t
    text = _C_TOKEN.sub(tok, open(path, encoding="utf-8").read())
    text = re.sub(r" +", " ", text).strip()
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def stored_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter summary,
    or None if absent or taken on different kernel code."""
    if not os.path.exists(PMC_SUMMARY):
        return None, None
    vals = {}
    for line in open(PMC_SUMMARY):
        if ":" in line and not line.startswith("#"):
            k_, _, v_ = line.partition(":")
            vals[k_.strip()] = v_.strip()
    if vals.get("kernel_code_sha256_16") != code_hash(KERNEL_SRC) or \
            vals.get("helpers_code_sha256_16") != code_hash(KERNEL_HDR):
        return None, vals
    try:
        return float(vals["hbm_bytes_per_launch"]), vals
    except (KeyError, ValueError):
        return None, vals


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=100, help="per-kernel timed calls")
    ap.add_argument("--profile", choices=["attn", "union", "copy", "compact", "prefill", "select"],
                    default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-prefill", action="store_true", help="skip the 64-chunk prefill leg")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the 64-chunk prefill leg and print its JSON object")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the leg that measures every config (1-5)")
    ap.add_argument("--config-oracle-seconds", type=float, default=120.0,
                    help="host time the configs leg may spend timing the oracle")
    ap.add_argument("--table", metavar="JSON",
                    help="print BASELINE.md's per-config table from a bench JSON line (a file "
                         "holding the line, or a driver record with it in its stdout tail) and exit")
    args = ap.parse_args()

    if args.table:
        print(markdown_table(_bench_line(json.load(open(args.table)))))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import gen
    import chunked_prefill_sparse_amd as ca

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.profile == "copy":
        n = 1 << 30  # 1 GiB
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for i in range(3):
            dst.copy_(src)
            torch.cuda.synchronize()
            log(f"copy {i}: {n} bytes")
        return

    if args.profile == "prefill":
        prefill_leg(stream, overlap=False)
        return
    if args.profile == "select":
        select_profile_leg(args.steps)
        return
    if args.prefill_only:
        print(json.dumps(prefill_leg(stream)))
        return

    log(f"generating {WORKLOAD} (pairwise mask) ...")
    w = gen.make_workload(WORKLOAD, variant="pairwise")
    variants = {"pairwise": w}
    for vname in ("dense", "colshared", "groupshared"):
        wv = gen.make_workload(WORKLOAD, variant=vname, with_tensors=False)
        wv.q, wv.k, wv.v = w.q, w.k, w.v
        variants[vname] = wv
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    out = torch.empty_like(q)
    masks = {n_: torch.from_numpy(x.mask).to(dev) for n_, x in variants.items()}
    torch.cuda.synchronize()

    def tables(name):
        x = variants[name]
        return ca.build_union_tables(masks[name], x.H_kv, x.n_q_blocks, x.n_kv_blocks)

    def attn(T, lens):
        return ca.chunk_attention(q, k, v, T, lens, w.prior, w.chunk, w.scale, out=out)

    bal_ws = torch.empty(ca.balanced_workspace_size(w.B, w.H_q, w.H_kv, w.C_max, w.D),
                         dtype=torch.uint8, device=dev)

    def attn_balanced(T, lens):
        return ca.chunk_attention(q, k, v, T, lens, w.prior, w.chunk, w.scale, out=out,
                                  balanced=True, workspace=bal_ws)

    if args.profile in ("attn", "union", "compact"):
        T, lens = tables("pairwise")
        if args.profile == "compact":
            k_out, v_out, T_out = ca.compact_kv(k, v, T, lens, w.prior, w.chunk)
        for i in range(max(args.steps, 1)):
            if args.profile == "attn":
                attn(T, lens)
            elif args.profile == "compact":
                ca.compact_kv(k, v, T, lens, w.prior, w.chunk, k_out, v_out, T_out)
            else:
                tables("pairwise")
            torch.cuda.synchronize()
            log(f"{args.profile} launch {i}")
        return

    results = {}
    for name in ("pairwise", "dense", "colshared", "groupshared"):
        x = variants[name]
        T, lens = tables(name)
        torch.cuda.synchronize()
        Th, lh = T.cpu().numpy(), lens.cpu().numpy()
        flops, bytes_alg, pairs = algorithmic(x, Th, lh)

        def step():
            T_, l_ = tables(name)
            attn(T_, l_)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
        attn_ms = time_calls(lambda: attn(T, lens), args.reps, stream)
        attn_bal_ms = time_calls(lambda: attn_balanced(T, lens), args.reps, stream)
        union_ms = time_calls(lambda: tables(name), args.reps, stream)
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold_ms = time_calls_cold(lambda: attn(T, lens), max(args.reps // 5, 5), stream, scratch)
        del scratch
        a_med = statistics.median(attn_ms)
        a_mean = float(np.mean(attn_ms))
        per_head_union = float(x.mask[:, :, :, :].any(axis=2).sum(axis=-1).mean())
        results[name] = dict(
            ms_per_step=ms_step,
            attn_ms_median=a_med, attn_ms_mean=a_mean,
            attn_ms_p10=pct(attn_ms, 10), attn_ms_p90=pct(attn_ms, 90),
            attn_ms_cold_median=statistics.median(cold_ms),
            union_us_median=statistics.median(union_ms) * 1e3,
            flops=flops, bytes_alg=bytes_alg, pairs=pairs,
            eff_tflops_step=flops / (ms_step * 1e-3) / 1e12,
            eff_tflops_attn=flops / (a_med * 1e-3) / 1e12,
            attn_balanced_ms_median=statistics.median(attn_bal_ms),
            eff_tflops_attn_balanced=flops / (statistics.median(attn_bal_ms) * 1e-3) / 1e12,
            mfma_frac_attn=flops / (a_mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            union_blocks_sum=int(lh.sum()), union_blocks_mean=float(lh.mean()),
            per_head_qunion_blocks_mean=per_head_union,
        )
        log(f"{name}: step {ms_step:.3f} ms, attention {a_med:.3f} ms "
            f"({results[name]['eff_tflops_attn']:.0f} TFLOP/s), balanced "
            f"{results[name]['attn_balanced_ms_median']:.3f} ms, union "
            f"{results[name]['union_us_median']:.1f} us, mean len {lh.mean():.0f}")
    # Explicit-compaction baseline: gather the selected blocks, then run the same
    # kernel on the compact buffer; zero-copy execution skips the gather.
    compaction = {}
    k_out, v_out = torch.empty_like(k), torch.empty_like(v)
    for name in ("pairwise", "colshared"):
        T, lens = tables(name)
        k_out, v_out, T_out = ca.compact_kv(k, v, T, lens, w.prior, w.chunk, k_out, v_out)
        torch.cuda.synchronize()
        blocks = int(lens.sum())
        copy_ms = time_calls(lambda: ca.compact_kv(k, v, T, lens, w.prior, w.chunk, k_out,
                                                   v_out, T_out), args.reps, stream)
        attn_c_ms = time_calls(lambda: ca.chunk_attention(q, k_out, v_out, T_out, lens, w.prior,
                                                          w.chunk, w.scale, out=out),
                               args.reps, stream)
        c_med, a_med = statistics.median(copy_ms), statistics.median(attn_c_ms)
        moved = 2 * 2 * blocks * 64 * w.D * 2  # K and V, read once and written once
        zc = results[name]["attn_ms_median"]
        compaction[name] = dict(
            copy_ms=round(c_med, 4), copy_GBps=round(moved / (c_med * 1e-3) / 1e9, 1),
            attn_ms_compact=round(a_med, 4), attn_ms_zero_copy=round(zc, 4),
            x_zero_copy_vs_compaction=round((c_med + a_med) / zc, 4))
        log(f"{name}: compaction copy {c_med:.3f} ms ({compaction[name]['copy_GBps']:.0f} GB/s), "
            f"attention on compact {a_med:.3f} ms, zero-copy {zc:.3f} ms")

    # Block-sparse-kernel baseline: each Q-block of each head attends its own
    # mask row (per-row lists, no union); also the same kernel fed the union as
    # every row's list, which does the union's work in the per-Q-block layout.
    sparse = {}
    for name in ("pairwise", "colshared", "groupshared"):
        x = variants[name]
        Tr, lr = ca.build_row_tables(masks[name], x.n_kv_blocks)
        torch.cuda.synchronize()
        pairs_rows = admissible_pairs_rows(x.mask, x.prior, x.chunk)
        flops_rows = 4 * w.D * pairs_rows
        rows_ms = time_calls(lambda: ca.chunk_attention_rows(q, k, v, Tr, lr, w.prior, w.chunk,
                                                             w.scale, out=out),
                             args.reps, stream)
        build_ms = time_calls(lambda: ca.build_row_tables(masks[name], x.n_kv_blocks, Tr, lr),
                              args.reps, stream)
        T, lens = tables(name)
        G, NQ = x.G, x.mask.shape[2]
        Tw = T.repeat_interleave(G, dim=1)[:, :, None, :].expand(-1, -1, NQ, -1).contiguous()
        lw = lens.repeat_interleave(G, dim=1)[:, :, None].expand(-1, -1, NQ).contiguous()
        wide_ms = time_calls(lambda: ca.chunk_attention_rows(q, k, v, Tw, lw, w.prior, w.chunk,
                                                             w.scale, out=out),
                             args.reps, stream)
        r_med, b_med, w_med = (statistics.median(rows_ms), statistics.median(build_ms),
                               statistics.median(wide_ms))
        u = results[name]
        sparse[name] = dict(
            attn_ms=round(r_med, 4), lists_us=round(b_med * 1e3, 2),
            eff_tflops=round(flops_rows / (r_med * 1e-3) / 1e12, 1),
            flops_frac_of_union=round(flops_rows / u["flops"], 4),
            mean_list_blocks=round(float(lr.float().mean()), 1),
            union_lists_attn_ms=round(w_med, 4),
            union_lists_eff_tflops=round(u["flops"] / (w_med * 1e-3) / 1e12, 1),
            x_union_kernel_vs_rows_kernel_same_work=round(w_med / u["attn_ms_median"], 4),
            x_union_vs_sparse=round((r_med + b_med) / (u["attn_ms_median"] + u["union_us_median"] * 1e-3), 4))
        log(f"{name}: sparse rows {r_med:.3f} ms ({sparse[name]['eff_tflops']:.0f} TFLOP/s, "
            f"{sparse[name]['flops_frac_of_union']:.3f} of the union's work); rows kernel on the "
            f"union lists {w_med:.3f} ms ({sparse[name]['union_lists_eff_tflops']:.0f} TFLOP/s)")
        del Tw, lw

    for name in results:
        results[name]["x_vs_dense_attn"] = results["dense"]["attn_ms_median"] / results[name]["attn_ms_median"]
        results[name]["x_vs_dense_step"] = results["dense"]["ms_per_step"] / results[name]["ms_per_step"]

    main_r = results["pairwise"]
    traffic, pmc = stored_traffic()
    achieved = main_r["flops"] / (main_r["attn_ms_mean"] * 1e-3) / 1e12
    # the shader clock the attention kernel ran at, from its own per-workgroup
    # records (real-time ticks and shader cycles), over 20 calls after the timed ones
    T, lens = tables("pairwise")
    stamps = None
    clocks = []
    for _ in range(20):
        _, stamps = ca.chunk_attention_stamped(q, k, v, T, lens, w.prior, w.chunk, w.scale,
                                               out=out, stamps=stamps)
        torch.cuda.synchronize()
        clocks.append(ca.stamps_summary(stamps))
    clock = statistics.median(c["clock_GHz"] for c in clocks)
    by_xcc = {x: round(statistics.median(c["clock_GHz_by_xcc"][x] for c in clocks), 3)
              for x in clocks[-1]["clock_GHz_by_xcc"]}
    log(f"shader clock during attention: {clock:.3f} GHz (by XCC {by_xcc})")
    roofline = {
        "bound": "mfma",
        "kernel": "chunk_attn_bf16_kernel<128, 8, false, 0>",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
        "alg_bytes": main_r["bytes_alg"],
        "hbm_alg_GBps": round(main_r["bytes_alg"] / (main_r["attn_ms_mean"] * 1e-3) / 1e9, 1),
        "hbm_frac": (round(traffic / (main_r["attn_ms_mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
                     if traffic else None),
        "reread_factor": round(traffic / main_r["bytes_alg"], 4) if traffic else None,
        "clock_GHz": round(clock, 4),
        "clock_GHz_by_xcc": by_xcc,
        "peak_at_clock": round(PEAK_BF16_TFLOPS * clock / PEAK_CLOCK_GHZ, 1),
        "frac_at_clock": round(achieved / (PEAK_BF16_TFLOPS * clock / PEAK_CLOCK_GHZ), 4),
    }
    del k_out, v_out
    configs = None
    if not args.no_configs:
        configs = configs_leg(stream, max(args.reps // 2, 20), w, (q, k, v), results,
                              args.config_oracle_seconds)
    tp_shard = tp_shard_leg(stream, args.reps)
    prefill = None if args.no_prefill else prefill_leg(stream)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, args.cpu_seconds)

    line = {
        "metric": "chunk attention eff. TFLOP/s at 128K ctx, LLaMA-8B GQA (union build + attention per step); x vs dense",
        "value": round(main_r["eff_tflops_step"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama8b_128k: B=1, H_q=32, H_kv=8, D=128, 129024 prior + 2048-token chunk, "
                        "block 64, mask sink + last 8 prior blocks + Bernoulli(0.05) per "
                        "(head, Q-block, KV-block)",
            "global_batch": 1, "seq_len": 131072, "parallelism": "none (1 GPU)",
        },
        "attn_ms": round(main_r["attn_ms_median"], 4),
        "union_us": round(main_r["union_us_median"], 2),
        "x_vs_dense": round(main_r["x_vs_dense_step"], 4),
        "variants": {n_: {k_: (round(v_, 4) if isinstance(v_, float) else v_) for k_, v_ in r.items()}
                     for n_, r in results.items()},
        "compaction": compaction,
        "block_sparse": sparse,
        "configs": configs,
        "tp_shard_128k": tp_shard,
        "prefill_128k": prefill,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
