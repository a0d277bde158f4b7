"""The library inside HIP graphs and on several streams.

It allocates nothing, never synchronises and records no memset, so its calls
can be captured into a HIP graph (torch.cuda.CUDAGraph) with preallocated
outputs and workspace.  Each graph is replayed several times, with eager
work and synchronisations in between, and every replay must give the eager
result bit for bit.  Calls enqueued on two streams at once (default
priority) must each give the single-stream result.
"""
import numpy as np
import pytest
import torch

import bf16_forward_attention_amd as attn
from bf16_forward_attention_amd import synth
from tests.gpu_util import say, to_bits, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


def _call(q, k, v, o, lse, ws, ws_bytes, B, H, H_kv, Sq, Sk, mode, mask, stream):
    st = attn.attn_fwd_bf16_gqa_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr() if lse is not None else 0, B, H, H_kv, Sq, Sk,
                                   attn.LAYOUTS["bshd"], attn.ROUND_MODES[mode], attn.MASKS[mask],
                                   ws.data_ptr() if ws is not None else 0, ws_bytes, stream.cuda_stream)
    if st != 0:
        raise attn.AttnError(st)


# (B, H, H_kv, Sq, Sk, mask): a key-range split (two kernels per call), a causal single pass
@pytest.mark.parametrize("shape", [(1, 4, 2, 300, 2000, "causal_br"), (2, 8, 8, 600, 700, "causal"),
                                   (1, 2, 2, 300, 3000, "none")], ids=lambda s: "x".join(map(str, s[:5])) + s[5])
def test_graph_replays_match_eager(shape):
    B, H, H_kv, Sq, Sk, mask = shape
    inp = synth.small(B, H, Sq, Sk, "bshd", seed=17, mask=mask, H_kv=H_kv)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    ws_bytes = attn.attn_fwd_bf16_gqa_workspace_size(B, H, Sq, Sk, attn.MASKS[mask])
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda:0")
    o_eager = torch.empty_like(q)
    lse_eager = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda:0")
    _call(q, k, v, o_eager, lse_eager, ws, ws_bytes, B, H, H_kv, Sq, Sk, "rtna", mask, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref_o, ref_lse = to_bits(o_eager), lse_eager.cpu().numpy().view(np.uint32)

    o = torch.zeros_like(q)
    lse = torch.zeros((B, H, Sq), dtype=torch.float32, device="cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up call on the capture stream, as torch recommends
        _call(q, k, v, o, lse, ws, ws_bytes, B, H, H_kv, Sq, Sk, "rtna", mask, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(q, k, v, o, lse, ws, ws_bytes, B, H, H_kv, Sq, Sk, "rtna", mask, torch.cuda.current_stream())
    for r in range(4):
        o.zero_()
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(o), ref_o), f"replay {r}: output differs from the eager call"
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), ref_lse), f"replay {r}: lse differs"
        # eager work between replays, on the same buffers
        _call(q, k, v, o, None, ws, ws_bytes, B, H, H_kv, Sq, Sk, "rtz", mask, torch.cuda.current_stream())
        torch.cuda.synchronize()
    say(f"  {shape}: 4 replays identical to the eager call (workspace {ws_bytes} B)")


def test_two_streams_at_once():
    B, H, Sq, Sk = 1, 8, 1000, 1500
    a = synth.small(B, H, Sq, Sk, "bshd", seed=21)
    b = synth.small(B, H, Sq, Sk, "bshd", seed=22, mask="causal")
    qa, ka, va = to_device(a.q), to_device(a.k), to_device(a.v)
    qb, kb, vb = to_device(b.q), to_device(b.k), to_device(b.v)
    ref_a, ref_b = torch.empty_like(qa), torch.empty_like(qb)
    # one workspace per stream: calls that share one must be ordered on a single stream
    na = attn.attn_fwd_bf16_gqa_workspace_size(B, H, Sq, Sk, attn.MASKS["none"])
    nb = attn.attn_fwd_bf16_gqa_workspace_size(B, H, Sq, Sk, attn.MASKS["causal"])
    assert na > 0  # the unmasked call splits its key ranges: two kernels per call
    wa = torch.empty(max(na, 16), dtype=torch.uint8, device="cuda:0")
    wb = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda:0")
    cur = torch.cuda.current_stream()
    _call(qa, ka, va, ref_a, None, wa, na, B, H, H, Sq, Sk, "rtne", "none", cur)
    _call(qb, kb, vb, ref_b, None, wb, nb, B, H, H, Sq, Sk, "rtne", "causal", cur)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a = [torch.empty_like(qa) for _ in range(3)]
    outs_b = [torch.empty_like(qb) for _ in range(3)]
    for oa, ob in zip(outs_a, outs_b):
        _call(qa, ka, va, oa, None, wa, na, B, H, H, Sq, Sk, "rtne", "none", s1)
        _call(qb, kb, vb, ob, None, wb, nb, B, H, H, Sq, Sk, "rtne", "causal", s2)
    torch.cuda.synchronize()
    for oa, ob in zip(outs_a, outs_b):
        assert np.array_equal(to_bits(oa), to_bits(ref_a))
        assert np.array_equal(to_bits(ob), to_bits(ref_b))
