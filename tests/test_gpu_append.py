"""GPU parity of ca_append_kv (the append step of chunked prefill) against
its oracle, bit for bit: a copy has exactly one right answer.  Every row
outside the appended ranges must keep its value (the caches start poisoned
with NaN there)."""
import numpy as np
import pytest
import torch

import chunked_prefill_sparse_amd as ca
from oracle import append_kv_ref
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.float32, 128), (torch.float32, 64)])
def test_append_matches_oracle(dtype, D):
    B, H_kv, C_max, L = 3, 2, 320, 1024
    prior, chunk = [0, 448, 700], [320, 64, 1]  # ragged, unaligned offsets too
    g = torch.Generator().manual_seed(91)
    kn = torch.randn((B, H_kv, C_max, D), generator=g).to(dtype)
    vn = torch.randn((B, H_kv, C_max, D), generator=g).to(dtype)
    kc = torch.full((B, H_kv, L, D), float("nan"), dtype=dtype)
    vc = torch.full((B, H_kv, L, D), float("nan"), dtype=dtype)
    say(f"append {dtype} D={D} prior={prior} chunk={chunk}")
    kd, vd = kc.cuda(), vc.cuda()
    ca.append_kv(kn.cuda(), vn.cuda(), kd, vd, prior, chunk)
    torch.cuda.synchronize()
    to = (lambda t: t.float().numpy()) if dtype == torch.bfloat16 else (lambda t: t.numpy())
    kr, vr = append_kv_ref(to(kc), to(vc), to(kn), to(vn), prior, chunk)
    for got, ref in ((kd, kr), (vd, vr)):
        np.testing.assert_array_equal(to(got.cpu()), ref)  # NaN == NaN here


def test_append_rebuilds_the_prompt():
    # a 2048-token prompt appended chunk by chunk equals the prompt itself
    B, H_kv, D, C, L = 1, 8, 128, 256, 2048
    full_k = torch.randn((B, H_kv, L, D)).to(torch.bfloat16).cuda()
    full_v = torch.randn((B, H_kv, L, D)).to(torch.bfloat16).cuda()
    kc = torch.zeros_like(full_k)
    vc = torch.zeros_like(full_v)
    for c in range(L // C):
        ca.append_kv(full_k[:, :, c * C:(c + 1) * C].contiguous(),
                     full_v[:, :, c * C:(c + 1) * C].contiguous(), kc, vc, [c * C], [C])
    torch.cuda.synchronize()
    assert torch.equal(kc, full_k) and torch.equal(vc, full_v)
