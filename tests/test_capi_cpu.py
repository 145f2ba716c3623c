"""The C-ABI library loads and exports every symbol declared in include/*.h, and
its host-side argument checks return the documented status codes.  Only calls
that fail validation are made here (they return before any HIP call), so no
GPU is needed."""
import ctypes
import glob
import os
import re

import pytest

from chunked_prefill_sparse_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        names |= set(re.findall(r"CA_EXPORT\s+[\w\s\*]+?\b(ca_\w+)\s*\(", text))
    return names


def test_header_declares_the_boundary():
    assert _declared_symbols() == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    for name in _declared_symbols():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = _lib.lib()
    for s in range(7):
        assert lib.ca_status_string(s).decode().startswith("CA_")
    assert lib.ca_status_string(99).decode() == "unknown ca_status"
    assert lib.ca_last_hip_error().decode() == ""


def _ints(*v):
    return (ctypes.c_int32 * len(v))(*v)


FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,status", [
    # mask, B, H_q, H_kv, NQ_max, NKB_max, nq, nkb, T, len
    ((None, 1, 4, 1, 1, 4, _ints(1), _ints(4), FAKE, FAKE), 1),
    ((FAKE, 1, 4, 1, 1, 4, _ints(1), _ints(4), None, FAKE), 1),
    ((FAKE, 1, 4, 1, 1, 4, None, _ints(4), FAKE, FAKE), 1),
    ((FAKE, 0, 4, 1, 1, 4, _ints(1), _ints(4), FAKE, FAKE), 2),
    ((FAKE, 129, 4, 1, 1, 4, _ints(1), _ints(4), FAKE, FAKE), 2),
    ((FAKE, 1, 4, 3, 1, 4, _ints(1), _ints(4), FAKE, FAKE), 2),
    ((FAKE, 1, 4, 1, 1, 4, _ints(2), _ints(4), FAKE, FAKE), 2),
    ((FAKE, 1, 4, 1, 1, 4, _ints(1), _ints(5), FAKE, FAKE), 2),
    ((FAKE, 1, 4, 1, 1, 4, _ints(-1), _ints(4), FAKE, FAKE), 2),
    ((FAKE, 1, 4, 1, 1, 1 << 20, _ints(1), _ints(4), FAKE, FAKE), 2),
])
def test_union_validation(args, status):
    lib = _lib.lib()
    assert lib.ca_build_union_tables(*args, None) == status


def _attn(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, T=FAKE, len=FAKE, NKB_max=20, prior=_ints(1024),
             chunk=_ints(256), B=1, H_q=4, H_kv=1, C_max=256, L=1280, D=64, block=64,
             scale=0.125, dtype=0, O=FAKE, lse=None)
    a.update(kw)
    return lib.ca_chunk_attention(a["Q"], a["K"], a["V"], a["T"], a["len"], a["NKB_max"],
                                  a["prior"], a["chunk"], a["B"], a["H_q"], a["H_kv"],
                                  a["C_max"], a["L"], a["D"], a["block"], a["scale"],
                                  a["dtype"], a["O"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), 1), (dict(K=None), 1), (dict(O=None), 1), (dict(prior=None), 1),
    (dict(dtype=7), 3),
    (dict(B=0), 2), (dict(H_kv=3), 2), (dict(scale=0.0), 2), (dict(scale=float("inf")), 2),
    (dict(chunk=_ints(512)), 2),               # chunk > C_max
    (dict(L=1000), 2),                         # prior + chunk > L
    (dict(NKB_max=10), 2),                     # table too short for the sequence
    (dict(prior=_ints(-64)), 2),
    (dict(D=96), 4), (dict(block=32), 4),
    (dict(prior=_ints(1000)), 4),              # unaligned prior
    (dict(chunk=_ints(250)), 4),               # unaligned chunk
    (dict(Q=FAKE + 8), 4),                     # not 16-byte aligned
    (dict(lse=FAKE + 2), 4),
    (dict(dtype=1, L=1 << 24, D=128), 4),      # bf16 cache slice of 4 GiB: beyond 32-bit offsets
])
def test_attention_validation(kw, status):
    assert _attn(_lib.lib(), **kw) == status


@pytest.mark.parametrize("args,status", [
    ((None, FAKE, 1, 8, 16, 1024, FAKE, FAKE), 1),
    ((FAKE, FAKE, 1, 8, 16, 1000, FAKE, FAKE), 2),   # L not a multiple of 64
    ((FAKE, FAKE, 1, 8, 32, 1024, FAKE, FAKE), 2),   # NKB_max > pages
    ((FAKE, FAKE, 0, 8, 16, 1024, FAKE, FAKE), 2),
])
def test_csr_validation(args, status):
    assert _lib.lib().ca_tables_to_csr(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((None, FAKE, 1, 8, 16, _ints(16), FAKE), 1),
    ((FAKE, FAKE, 1, 8, 16, None, FAKE), 1),
    ((FAKE, FAKE, 1, 8, 16, _ints(16), None), 1),
    ((FAKE, FAKE, 0, 8, 16, _ints(16), FAKE), 2),
    ((FAKE, FAKE, 1, 0, 16, _ints(16), FAKE), 2),
    ((FAKE, FAKE, 1, 8, 16, _ints(17), FAKE), 2),    # n_kv_blocks > NKB_max
    ((FAKE, FAKE, 1, 8, 16, _ints(-1), FAKE), 2),
])
def test_check_tables_validation(args, status):
    assert _lib.lib().ca_check_tables(*args, None) == status


def _compact(lib, **kw):
    a = dict(K=FAKE, V=FAKE, T=FAKE, len=FAKE, NKB_max=20, prior=_ints(1024), chunk=_ints(256),
             B=1, H_kv=1, L=1280, D=64, dtype=1, Ko=FAKE, Vo=FAKE, To=FAKE)
    a.update(kw)
    return lib.ca_compact_kv(a["K"], a["V"], a["T"], a["len"], a["NKB_max"], a["prior"],
                             a["chunk"], a["B"], a["H_kv"], a["L"], a["D"], a["dtype"], a["Ko"],
                             a["Vo"], a["To"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=None), 1), (dict(Vo=None), 1), (dict(To=None), 1), (dict(chunk=None), 1),
    (dict(dtype=9), 3),
    (dict(B=0), 2), (dict(B=129), 2), (dict(H_kv=0), 2),
    (dict(L=1000), 2),                         # prior + chunk > L
    (dict(NKB_max=19), 2),                     # table too short for the sequence
    (dict(prior=_ints(-64)), 2),
    (dict(D=80), 4), (dict(prior=_ints(1000)), 4), (dict(Ko=FAKE + 4), 4),
])
def test_compact_validation(kw, status):
    assert _compact(_lib.lib(), **kw) == status


def test_rows_validation():
    lib = _lib.lib()
    base = (FAKE, FAKE, FAKE, FAKE, FAKE)
    # NQ_max * 64 must cover C_max
    assert lib.ca_chunk_attention_rows(*base, 3, 20, _ints(1024), _ints(256), 1, 4, 1, 256, 1280,
                                       64, 64, 0.125, 1, FAKE, None, None) == 2
    assert lib.ca_chunk_attention_rows(*base, 4, 20, _ints(1024), _ints(256), 1, 4, 1, 256, 1280,
                                       96, 64, 0.125, 1, FAKE, None, None) == 4
    assert lib.ca_chunk_attention_rows(None, *base[1:], 4, 20, _ints(1024), _ints(256), 1, 4, 1,
                                       256, 1280, 64, 64, 0.125, 1, FAKE, None, None) == 1


def test_split_validation_and_workspace_size():
    lib = _lib.lib()
    assert lib.ca_chunk_attention_workspace_size(1, 4, 2048, 128, 4) == 4 * 4 * 2048 * 130 * 4
    assert lib.ca_chunk_attention_workspace_size(1, 4, 2048, 128, 1) == 0
    base = (FAKE, FAKE, FAKE, FAKE, FAKE, 20, _ints(1024), _ints(256), 1, 4, 1, 256, 1280, 64, 64,
            0.125)
    need = lib.ca_chunk_attention_workspace_size(1, 4, 256, 64, 4)
    # too many splits, fp32 split with a short workspace, no workspace, short workspace,
    # unaligned workspace
    assert lib.ca_chunk_attention_split(*base, 1, 17, FAKE, need, FAKE, None, None) == 2
    assert lib.ca_chunk_attention_split(*base, 0, 4, FAKE, need - 1, FAKE, None, None) == 2
    assert lib.ca_chunk_attention_split(*base, 1, 4, None, need, FAKE, None, None) == 1
    assert lib.ca_chunk_attention_split(*base, 1, 4, FAKE, need - 1, FAKE, None, None) == 2
    assert lib.ca_chunk_attention_split(*base, 1, 4, FAKE + 4, need, FAKE, None, None) == 4


def test_balanced_validation_and_workspace_size():
    lib = _lib.lib()
    # parts = 2 * tiles + 1024 partial tiles of 256 rows (D floats, then 2 floats per row), then
    # the part numbering, tiles + 1 ints (tiles = B * H_kv * ceil(G * ceil(C_max / 32) / 8)),
    # each part 16-byte aligned
    tiles = 1 * 8 * ((4 * 64 + 7) // 8)
    parts = 2 * tiles + 1024
    up16 = lambda x: (x + 15) // 16 * 16
    want = up16(up16(up16(parts * 256 * 128 * 4) + parts * 256 * 2 * 4) + (tiles + 1) * 4)
    assert lib.ca_chunk_attention_balanced_workspace_size(1, 32, 8, 2048, 128) == want
    # more than 1024 tiles: the plain kernel runs, no workspace is used
    assert lib.ca_chunk_attention_balanced_workspace_size(5, 32, 8, 2048, 64) == 16
    assert lib.ca_chunk_attention_balanced_workspace_size(1, 32, 7, 2048, 128) == 0
    assert lib.ca_chunk_attention_balanced_workspace_size(1, 32, 8, 2048, 80) == 0
    assert lib.ca_chunk_attention_balanced_workspace_size(0, 32, 8, 2048, 128) == 0
    base = (FAKE, FAKE, FAKE, FAKE, FAKE, 20, _ints(1024), _ints(256), 1, 4, 1, 256, 1280, 64, 64,
            0.125)
    need = lib.ca_chunk_attention_balanced_workspace_size(1, 4, 1, 256, 64)
    # no workspace, short workspace, unaligned workspace, bad dtype, bad shape
    assert lib.ca_chunk_attention_balanced(*base, 1, None, need, FAKE, None, None) == 1
    assert lib.ca_chunk_attention_balanced(*base, 1, FAKE, need - 1, FAKE, None, None) == 2
    assert lib.ca_chunk_attention_balanced(*base, 1, FAKE + 4, need, FAKE, None, None) == 4
    assert lib.ca_chunk_attention_balanced(*base, 7, FAKE, need, FAKE, None, None) == 3
    bad = base[:10] + (3,) + base[11:]  # H_q = 4 over H_kv = 3
    assert lib.ca_chunk_attention_balanced(*bad, 1, FAKE, need, FAKE, None, None) == 2


def test_split_noalloc_validation():
    # Sizes past the static array and bad arguments are refused on the host,
    # before the array's address is looked up (no GPU is touched here).
    lib = _lib.lib()
    base = (FAKE, FAKE, FAKE, FAKE, FAKE, 20, _ints(1024), _ints(256), 1, 4, 1, 256, 1280, 64, 64,
            0.125)
    assert lib.ca_chunk_attention_split_noalloc(*base, 1, 17, FAKE, None, None) == 2
    assert lib.ca_chunk_attention_split_noalloc(*base, 1, 0, FAKE, None, None) == 2
    assert lib.ca_chunk_attention_split_noalloc(None, *base[1:], 1, 4, FAKE, None, None) == 1
    assert lib.ca_chunk_attention_split_noalloc(*base, 9, 4, FAKE, None, None) == 3
    assert lib.ca_chunk_attention_split_noalloc(*base[:13], 96, *base[14:], 1, 4, FAKE, None,
                                                None) == 4
    # one GPU's tensor-parallel share of a 2048-row chunk (4 heads, D = 128: 130 floats per
    # row and split) fits at 15 splits and not at 16
    cap = _lib.CA_STATIC_SCRATCH_BYTES
    assert lib.ca_chunk_attention_workspace_size(1, 4, 2048, 128, 15) == 15 * 4259840 <= cap
    assert lib.ca_chunk_attention_workspace_size(1, 4, 2048, 128, 16) > cap
    tp = (FAKE, FAKE, FAKE, FAKE, FAKE, 2048, _ints(129024), _ints(2048), 1, 4, 1, 2048,
          131072, 128, 64, 0.088)
    assert lib.ca_chunk_attention_split_noalloc(*tp, 1, 16, FAKE, None, None) == \
        _lib.CA_ERR_TOO_LARGE
    # the whole 32-head chunk fits no split at all (65 MiB at 2)
    big = tp[:9] + (32, 8) + tp[11:]
    assert lib.ca_chunk_attention_split_noalloc(*big, 1, 2, FAKE, None, None) == \
        _lib.CA_ERR_TOO_LARGE
    assert lib.ca_status_string(_lib.CA_ERR_TOO_LARGE).decode().startswith("CA_ERR_TOO_LARGE")


def test_devlen_validation():
    # the device-length calls check everything the host can see; their length
    # arrays are device pointers that the host never reads
    lib = _lib.lib()
    ua = lib.ca_build_union_tables_devlen
    assert ua(None, 1, 4, 1, 1, 4, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert ua(FAKE, 1, 4, 1, 1, 4, None, FAKE, FAKE, FAKE, None) == 1
    assert ua(FAKE, 0, 4, 1, 1, 4, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert ua(FAKE, 1, 4, 3, 1, 4, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert ua(FAKE, 1, 4, 1, 1, 1 << 20, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert ua(FAKE, 1, 4, 1, 1, 4, FAKE + 2, FAKE, FAKE, FAKE, None) == 4  # misaligned
    at = lib.ca_chunk_attention_devlen
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 20, FAKE, FAKE, 1, 4, 1, 256, 1280, 64, 64, 0.125, 1,
            FAKE, None, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return at(*a)

    assert call(a0=None) == 1 and call(a6=None) == 1 and call(a17=None) == 1
    assert call(a16=7) == 3
    assert call(a8=0) == 2 and call(a10=3) == 2 and call(a15=0.0) == 2
    assert call(a13=96) == 4 and call(a14=32) == 4
    assert call(a7=FAKE + 2) == 4  # misaligned device lengths
    assert call(a12=1 << 24, a13=128) == 4  # bf16 slice past 32-bit offsets


def test_append_validation():
    lib = _lib.lib()
    # K_new, V_new, B, H_kv, C_max, L, D, dtype, prior, chunk, K_cache, V_cache
    base = [FAKE, FAKE, 1, 2, 128, 1024, 64, 1, _ints(896), _ints(128), FAKE, FAKE]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.ca_append_kv(*a, None)

    assert call(a0=None) == 1 and call(a8=None) == 1 and call(a11=None) == 1
    assert call(a7=5) == 3
    assert call(a2=0) == 2 and call(a3=0) == 2
    assert call(a9=_ints(129)) == 2               # chunk > C_max
    assert call(a8=_ints(897)) == 2               # prior + chunk > L
    assert call(a8=_ints(-1)) == 2
    assert call(a6=96) == 4 and call(a10=FAKE + 8) == 4


def test_stamped_validation():
    lib = _lib.lib()
    n = ctypes.c_int(-1)
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 20, _ints(1024), _ints(256), 1, 4, 1, 256, 1280, 64, 64,
            0.125, 1, FAKE, None]
    st = lib.ca_chunk_attention_stamped
    assert st(*base, None, 16, ctypes.byref(n), None) == 1
    # no buffer: the count only (4 heads x 256 rows in 32-row tiles, 4 per workgroup)
    assert st(*base, None, 0, ctypes.byref(n), None) == 2 and n.value == 8
    assert st(*base, FAKE, 16, None, None) == 1
    assert st(*base[:16], 0, *base[17:], FAKE, 16, ctypes.byref(n), None) == 4  # fp32
    assert st(*base, FAKE + 2, 16, ctypes.byref(n), None) == 4
    assert st(*base[:6], _ints(1000), *base[7:], FAKE, 16, ctypes.byref(n), None) == 4


def test_select_chunk_validation():
    lib = _lib.lib()
    # Q, K, dtype, B, H_q, H_kv, C_max, L, D, prior, chunk, budget, local, qbar, NQ_max, kbar,
    # NKB_max, scores, mask, T, len
    base = [FAKE, FAKE, 1, 1, 8, 2, 256, 4096, 64, _ints(1024), _ints(256), 8, 2, FAKE, 4, FAKE,
            64, FAKE, FAKE, FAKE, FAKE]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.ca_select_chunk(*a, None)

    assert call(a0=None) == 1 and call(a18=None) == 1 and call(a20=None) == 1
    assert call(a2=3) == 3
    assert call(a5=3) == 2 and call(a11=-1) == 2 and call(a16=1 << 20) == 2
    assert call(a10=_ints(320)) == 2            # chunk > C_max
    assert call(a14=3) == 2                     # chunk > 64 * NQ_max
    assert call(a9=_ints(4096 - 128)) == 2      # prior + chunk > L
    assert call(a8=96) == 4 and call(a9=_ints(1000)) == 4 and call(a13=FAKE + 4) == 4
