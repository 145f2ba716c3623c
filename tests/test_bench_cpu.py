"""CPU checks of the benchmark's own arithmetic and contract.

* The work accounting behind the metric (admissible (query, key) pairs, hence
  the algorithmic FLOPs) against brute-force loops on tiny tables, for union
  execution and for block-sparse per-Q-block execution.
* The code hash that ties the stored counter summary to the kernel: blind to
  comments and white space, sensitive to code.
* One GPU only: ``--gpus 2`` exits with a message before touching a GPU.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from oracle import union_tables_ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _brute_pairs(T, lens, prior, chunk, G):
    n = 0
    for b in range(T.shape[0]):
        P, C = prior[b], chunk[b]
        for g in range(T.shape[1]):
            keys = [t for kb in T[b, g, :lens[b, g]] for t in range(64 * kb, 64 * kb + 64)]
            for i in range(C):
                n += G * sum(1 for t in keys if t <= P + i and t < P + C)
    return n


def _brute_pairs_rows(mask, prior, chunk):
    n = 0
    for b in range(mask.shape[0]):
        P, C = prior[b], chunk[b]
        for h in range(mask.shape[1]):
            for qb in range(C // 64):
                for kb in np.flatnonzero(mask[b, h, qb, :(P + C) // 64]):
                    for i in range(64 * qb, 64 * qb + 64):
                        n += sum(1 for t in range(64 * kb, 64 * kb + 64) if t <= P + i)
    return n


@pytest.mark.parametrize("seed", range(6))
def test_admissible_pairs_brute_force(seed):
    rng = np.random.default_rng(seed)
    B, H_kv, G = 2, 2, 2
    prior = [64 * int(rng.integers(0, 5)) for _ in range(B)]
    chunk = [64 * int(rng.integers(1, 4)) for _ in range(B)]
    nq = [c // 64 for c in chunk]
    nkb = [(p + c) // 64 for p, c in zip(prior, chunk)]
    NKB = max(nkb)
    mask = (rng.random((B, H_kv * G, max(nq), NKB)) < 0.4).astype(np.uint8)
    T, ln = union_tables_ref(mask, H_kv, nq, nkb)
    assert bench.admissible_pairs(T, ln, prior, chunk, G) == _brute_pairs(T, ln, prior, chunk, G)
    assert bench.admissible_pairs_rows(mask, prior, chunk) == _brute_pairs_rows(mask, prior, chunk)


def test_code_hash_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text('// one\nint f(int x) {  /* two */ return x + 1; }\nconst char* s = "// kept";\n')
    b = tmp_path / "b.hip"
    b.write_text('// changed\n\nint f(int x) {\n  return x + 1;  // three\n}\nconst char* s = "// kept";\n')
    c = tmp_path / "c.hip"
    c.write_text('int f(int x) { return x + 2; }\nconst char* s = "// kept";\n')
    d = tmp_path / "d.hip"
    d.write_text('int f(int x) { return x + 1; }\nconst char* s = "// other";\n')
    assert bench.code_hash(a) == bench.code_hash(b)
    assert bench.code_hash(a) != bench.code_hash(c)
    assert bench.code_hash(a) != bench.code_hash(d)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")


def test_blocks_summary_and_table():
    # the union-size summary of a tiny workload, by hand, and the per-config table
    import gen
    w = gen.make_custom(1, 4, 2, 64, [128], [128], "bf16", 3,
                        lambda rng, b, H, nq, pb: np.zeros((H, nq, pb), np.uint8),
                        with_tensors=False)
    w.mask[0, 0, 0, 0] = 1  # head 0 (group 0), Q-block 0 selects prior block 0
    T, ln = union_tables_ref(w.mask, w.H_kv, w.n_q_blocks, w.n_kv_blocks)
    # group 0: block 0 + the chunk's two blocks; group 1: the chunk's two blocks
    assert ln.tolist() == [[3, 2]]
    # per head: heads 0 sees {0, 2, 3}, the others {2, 3}
    assert bench.blocks_summary(w, ln) == [5, 2.5, 2.2, 4.0]
    rec = {"configs": {"tiny_f32": dict(cfg=1, dtype="f32", ms=[0.1, 0.09, 0.11],
                                        union_us=[10.0, 3.5], tflops=2.5, hbm_GBps=10.0,
                                        len=[19, 19.0, 14.0, 20.0], split8_ms=0.026,
                                        dense_ms=0.105, x_dense=1.05,
                                        oracle=dict(s=0.005, sample="whole", cores=16)),
                       "vslash_128k.d0.02.identical": dict(
                           cfg=5, dtype="bf16", ms=[1.0, 0.99, 1.01], union_us=[12.0, 9.0],
                           tflops=1200.0, hbm_GBps=180.0, mfma=0.48,
                           len=[4848, 606.0, 606.0, 2048.0, 0.0195], dense_ms=3.5, x_dense=3.5,
                           oracle=dict(s=None, sample="skipped"))}}
    table = bench.markdown_table(rec).splitlines()
    assert len(table) == 4
    assert table[2].startswith("| 1 tiny_f32 (fp32) | 0.100; 0.090–0.110 (8 splits: 0.026) |")
    assert "| 0.005 (16) |" in table[2] and "| — | 10 | 1.05 |" in table[2]
    assert table[3].startswith("| 5 vslash_128k d0.02.identical | 1.000;")
    assert table[3].endswith("| 606 / 606 / 2048 | — |")
    # a driver record holding the line in its stdout tail
    import json
    drv = {"parsed": {"value": 1}, "run": {"stdout_tail": json.dumps(rec) + "\n\n---- stderr"}}
    assert bench._bench_line(drv) == rec
