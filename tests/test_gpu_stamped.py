"""ca_chunk_attention_stamped: the same output as ca_chunk_attention, bit for
bit, plus one timing record per workgroup whose fields are consistent (every
workgroup recorded once, positive spans, a shader clock within the range a
GPU runs at, XCC ids of the chip)."""
import pytest
import torch

import gen
import chunked_prefill_sparse_amd as ca
from tests.gpu_util import Dev, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw", [("llama8b_32k", {}), ("ragged_b4", {})])
def test_stamped_matches_plain(name, kw):
    w = gen.make_workload(name, **kw)
    d = Dev(w)
    T, lens = d.tables()
    O = d.attention(T, lens)
    Os, stamps = ca.chunk_attention_stamped(d.q, d.k, d.v, T, lens, w.prior, w.chunk, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(O, Os)
    s = ca.stamps_summary(stamps)
    say(f"{name}: {s}")
    a = stamps.cpu()
    assert bool((a[:, 1] > 0).all()) and bool((a[:, 2] > 0).all())
    assert 0.3 <= s["clock_GHz"] <= 3.0
    assert all(0 <= x < 8 for x in s["clock_GHz_by_xcc"])
    assert s["workgroups"] == stamps.shape[0] > 0
