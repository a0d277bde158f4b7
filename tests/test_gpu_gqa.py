"""GPU parity of grouped-query attention (attn_fwd_bf16_gqa) against the oracle.

The reading (the pages list GQA only as missing from the kernel they
describe): K/V hold H_kv heads and query head h uses K/V head h / (H / H_kv).
Every row is compared under the row-scaled 2-ULP gate, with and without the
causal masks; the kernel on grouped heads must give exactly the bits it gives
with the K/V heads repeated (the same arithmetic on the same values).
"""
import numpy as np
import pytest
import torch

import oracle
from bf16_forward_attention_amd import synth
from tests.gate import gate
from tests.gpu_util import MODES, Dev, launch_masked, say, to_bits, to_device

pytestmark = pytest.mark.gpu

SHAPES = [(1, 8, 1, 300, 300), (2, 8, 2, 256, 513), (1, 6, 3, 700, 129), (1, 4, 4, 100, 64), (2, 16, 4, 513, 1000)]


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("mask", ["none", "causal", "causal_br"])
def test_gqa_shapes(shape, layout, mask):
    B, H, H_kv, Sq, Sk = shape
    inp = synth.small(B, H, Sq, Sk, layout, seed=H * 100 + H_kv + Sq, mask=mask, H_kv=H_kv)
    ex, rd = oracle.attn_all(inp.q, inp.k, inp.v, layout, mask=mask)
    dev = Dev(inp)
    for m, mode in enumerate(MODES):
        got = dev.run_logical(mode)
        res = gate(got, rd[m], ex)
        say(f"  {inp.wl.name} {mode}: {res.summary()}")
        assert res.ok, f"{inp.wl.name} {mode}: {res.summary()}"
    assert np.array_equal(dev.run_logical(MODES[0]), dev.run_logical(MODES[0])), "repeated launch changed the output"


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_grouped_heads_match_repeated_heads_bit_for_bit(layout, mask):
    B, H, H_kv, Sq, Sk = 2, 8, 2, 400, 700
    inp = synth.small(B, H, Sq, Sk, layout, seed=5, mask=mask, H_kv=H_kv)
    got = Dev(inp).run(MODES[1])
    axis = 2 if layout == "bshd" else 1
    k_rep = np.ascontiguousarray(np.repeat(inp.k, H // H_kv, axis=axis))
    v_rep = np.ascontiguousarray(np.repeat(inp.v, H // H_kv, axis=axis))
    q, k, v = to_device(inp.q), to_device(k_rep), to_device(v_rep)
    o = torch.empty_like(q)
    launch_masked(q, k, v, o, layout, MODES[1], mask)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(o), got)
