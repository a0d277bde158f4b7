"""GPU parity at the size limits of the argument checks.

The tile loads address the 64 K/V rows of a tile with 32-bit offsets, so the
head count is capped at 2^18 (in BSHD a K/V row is H * 256 bytes apart): at
the cap the last row of a tile sits 63 * 2^26 bytes from its first.  These
cases run the kernel right at the cap and compare sampled heads with the
oracle, which sees only those heads' slices.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gate import gate
from tests.gpu_util import launch, launch_gqa, say

pytestmark = pytest.mark.gpu

H_MAX = 1 << 18


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("H_kv", [H_MAX, 1])
def test_largest_head_count_bshd(H_kv):
    # B=1, Sq=3, Sk=64 (one full tile: rows 0..63 of every head), H = 2^18 query heads
    B, Sq, Sk, H = 1, 3, 64, H_MAX
    g = torch.Generator(device="cuda:0").manual_seed(7)
    q = torch.randn((B, Sq, H, 128), generator=g, device="cuda:0").to(torch.bfloat16)
    k = torch.randn((B, Sk, H_kv, 128), generator=g, device="cuda:0").to(torch.bfloat16)
    v = torch.randn((B, Sk, H_kv, 128), generator=g, device="cuda:0").to(torch.bfloat16)
    o = torch.empty_like(q)
    if H_kv == H:
        launch(q, k, v, o, "bshd", "rtne")
    else:
        launch_gqa(q, k, v, o, "bshd", "rtne")
    torch.cuda.synchronize()
    group = H // H_kv
    for h in (0, 1, 12345, H // 2 + 3, H - 2, H - 1):
        hk = h // group
        qs = np.ascontiguousarray(_bits(q[:, :, h:h + 1]))
        ks = np.ascontiguousarray(_bits(k[:, :, hk:hk + 1]))
        vs = np.ascontiguousarray(_bits(v[:, :, hk:hk + 1]))
        ex, rd = oracle.attn_rows(qs, ks, vs, "bshd", [(0, 0, i) for i in range(Sq)])
        got = np.ascontiguousarray(_bits(o[:, :, h])[0])
        res = gate(got[None], rd[None, :, 0], ex[None])
        say(f"  H_kv={H_kv} head {h}: {res.summary()}")
        assert res.ok, (h, res.summary())
