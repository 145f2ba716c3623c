"""Pins for the append oracle (CPU only).

Chunked prefill (problem statement of the technical summaries): each chunk's
keys and values go into the cache after the prior tokens before the chunk
attends.  A hand-worked case, the rebuild of a whole prompt chunk by chunk (in
any order), and the untouched rest of the cache pin the oracle.
"""
import numpy as np

from oracle import append_kv_ref


def test_hand_worked_case():
    # cache of 6 rows (D = 2) holding 100 + row; a 2-row chunk (C_max = 3, third
    # row unused) appended at prior = 3 replaces rows 3 and 4 only
    k = (100 + np.arange(6, dtype=np.float32))[None, None, :, None].repeat(2, axis=3)
    v = -k
    kn = np.array([[[[1, 2], [3, 4], [9, 9]]]], np.float32)
    vn = -kn
    ko, vo = append_kv_ref(k, v, kn, vn, [3], [2])
    assert ko[0, 0, :, 0].tolist() == [100, 101, 102, 1, 3, 105]
    assert ko[0, 0, :, 1].tolist() == [100, 101, 102, 2, 4, 105]
    np.testing.assert_array_equal(vo, -ko)
    assert k[0, 0, 3, 0] == 103  # the input is not modified


def test_rebuilds_a_prompt_in_any_order():
    rng = np.random.default_rng(5)
    B, H, L, D, C = 2, 3, 64 * 6, 8, 64 * 2
    full_k = rng.standard_normal((B, H, L, D)).astype(np.float32)
    full_v = rng.standard_normal((B, H, L, D)).astype(np.float32)
    for order in ([0, 1, 2], [2, 0, 1]):
        k = np.zeros_like(full_k)
        v = np.zeros_like(full_v)
        for c in order:
            kn = np.ascontiguousarray(full_k[:, :, c * C:(c + 1) * C])
            vn = np.ascontiguousarray(full_v[:, :, c * C:(c + 1) * C])
            k, v = append_kv_ref(k, v, kn, vn, [c * C] * B, [C] * B)
        np.testing.assert_array_equal(k, full_k)
        np.testing.assert_array_equal(v, full_v)


def test_empty_chunk_and_ragged_batch():
    k = np.arange(2 * 1 * 8 * 2, dtype=np.float32).reshape(2, 1, 8, 2)
    kn = -np.ones((2, 1, 4, 2), np.float32)
    ko, _ = append_kv_ref(k, k, kn, kn, [2, 5], [0, 3])
    np.testing.assert_array_equal(ko[0], k[0])          # empty chunk: unchanged
    assert (ko[1, 0, 5:8] == -1).all() and (ko[1, 0, :5] == k[1, 0, :5]).all()
