"""attn_fwd_bf16_gqa_noalloc: the split path on the library's static scratch.

It must give exactly the bits of attn_fwd_bf16_gqa_ws with a workspace of the
size the library asks for (the same plan and kernels), on two calls in a row,
the second smaller, so the second runs over the partials the first left in
the scratch; and both agree with the oracle under the gate.  The first shape
(few heads of a long causal sequence: every item cut into 8 key ranges, 512
partial blocks) fills the whole static array.
"""
import numpy as np
import pytest
import torch

import bf16_forward_attention_amd as attn
import oracle
from bf16_forward_attention_amd import synth
from tests.gate import gate
from tests.gpu_util import MODES, say, to_bits, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


def _call(entry, inp, mode, mask, lse):
    wl = inp.wl
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    o = torch.empty_like(q)
    s = torch.cuda.current_stream().cuda_stream
    lse_ptr = lse.data_ptr() if lse is not None else 0
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_ptr, wl.B, wl.H, wl.kv_heads, wl.Sq, wl.Sk,
            attn.LAYOUTS[wl.layout], attn.ROUND_MODES[mode], attn.MASKS[mask])
    if entry == "noalloc":
        st = attn.attn_fwd_bf16_gqa_noalloc(*args, s)
    else:
        nbytes = attn.attn_fwd_bf16_gqa_workspace_size(wl.B, wl.H, wl.Sq, wl.Sk, attn.MASKS[mask])
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda:0")
        st = attn.attn_fwd_bf16_gqa_ws(*args, ws.data_ptr(), nbytes, s)
    assert st == 0, attn.attn_fwd_bf16_strerror(st)
    torch.cuda.synchronize()
    return to_bits(o)


# (B, H, H_kv, Sq, Sk, layout, mask, mode): two calls in a row, the second smaller
CASES = [
    ((1, 4, 4, 4096, 4096, "bshd", "causal", "rtne"), (1, 2, 2, 300, 3000, "bhsd", "none", "rtz")),
    ((2, 8, 2, 300, 2000, "bshd", "causal_br", "rtna"), (1, 3, 1, 250, 700, "bshd", "causal_br", "rtne")),
]


@pytest.mark.parametrize("pair", CASES, ids=["long_causal_then_short", "gqa_bottom_right_then_smaller"])
def test_noalloc_matches_the_workspace_entry_point(pair):
    for B, H, H_kv, Sq, Sk, layout, mask, mode in pair:
        need = attn.attn_fwd_bf16_gqa_workspace_size(B, H, Sq, Sk, attn.MASKS[mask])
        assert need > 0, "the case must split its key ranges, or the scratch is not used"
        inp = synth.small(B, H, Sq, Sk, layout, seed=Sq + Sk, mask=mask, H_kv=H_kv)
        lse_a = torch.full((B, H, Sq), 7.0, dtype=torch.float32, device="cuda:0")
        lse_b = torch.full((B, H, Sq), -7.0, dtype=torch.float32, device="cuda:0")
        got = _call("noalloc", inp, mode, mask, lse_a)
        ref = _call("ws", inp, mode, mask, lse_b)
        say(f"  {B}x{H}x{H_kv} {Sq}x{Sk} {mask} {mode}: {need} B of partials")
        assert np.array_equal(got, ref), "noalloc and workspace entry points differ"
        assert torch.equal(lse_a, lse_b), "lse differs"
        again = _call("noalloc", inp, mode, mask, None)
        assert np.array_equal(again, got), "noalloc not deterministic"
        if Sq * Sk * B * H <= 2 * 10**8:
            ex, rd = oracle.attn_all(inp.q, inp.k, inp.v, layout, mask=mask)
            res = gate(np.ascontiguousarray(synth.to_logical(got, layout)), rd[MODES.index(mode)], ex)
            say(f"    oracle: {res.summary()}")
            assert res.ok, res.summary()


def test_noalloc_without_a_split_is_the_single_pass():
    # 64 heads x 4 q-tiles = 256 work items, a whole round of compute units: no split, the call is
    # attn_fwd_bf16_gqa
    inp = synth.small(1, 64, 1024, 300, "bshd", seed=3)
    assert attn.attn_fwd_bf16_gqa_workspace_size(1, 64, 1024, 300, 0) == 0
    got = _call("noalloc", inp, "rtne", "none", None)
    ref = _call("ws", inp, "rtne", "none", None)
    assert np.array_equal(got, ref)
