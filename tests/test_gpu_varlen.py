"""GPU parity of variable-length batches (attn_fwd_bf16_varlen) against the oracle.

Sequences are packed one after another (FlashAttention's cu_seqlens layout)
and each attends within itself.  Every row is compared under the row-scaled
2-ULP gate with identical NaN/Inf positions, and each sequence must give
exactly the bits the fixed-length entry point gives for it alone (the same
arithmetic on the same rows).
"""
import numpy as np
import pytest
import torch

import bf16_forward_attention_amd as attn
import oracle
from bf16_forward_attention_amd import synth
from tests.gate import gate
from tests.gpu_util import MODES, launch_gqa, say, to_bits, to_device

pytestmark = pytest.mark.gpu

CASES = [
    # (lengths_q, lengths_k, H, H_kv)
    ((1,), (1,), 2, 2),
    ((300, 17, 1024, 1, 513), (300, 17, 1024, 1, 513), 4, 2),
    ((64, 256, 257, 700), (1000, 65, 3, 700), 8, 8),
    ((0, 100, 0, 40), (50, 0, 0, 40), 4, 1),   # empty queries, keys-less sequence, empty both
    ((1200,), (33,), 2, 1),
]


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


def _run(inp, mode, mask, max_q=None):
    wl = inp.wl
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    cq = torch.from_numpy(inp.cu_q).to("cuda:0")
    ck = torch.from_numpy(inp.cu_k).to("cuda:0")
    o = torch.full_like(q, float("nan"))
    st = attn.attn_fwd_bf16_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), 0, cq.data_ptr(),
                                   ck.data_ptr(), wl.B, wl.H, wl.H_kv, q.shape[0], k.shape[0],
                                   max_q or max(max(wl.lengths_q), 1), attn.ROUND_MODES[mode], attn.MASKS[mask],
                                   torch.cuda.current_stream().cuda_stream)
    if st != 0:
        raise attn.AttnError(st)
    torch.cuda.synchronize()
    return to_bits(o)


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("mask", ["none", "causal", "causal_br"])
def test_varlen_all_rows(case, mask):
    lq, lk, H, H_kv = CASES[case]
    wl = synth.VarlenWorkload(f"varlen{case}", lq, lk, H, H_kv, MODES, mask=mask, seed=case + 11)
    inp = synth.generate_varlen(wl)
    ex, rd = oracle.attn_all_varlen(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, mask)
    for m, mode in enumerate(MODES):
        got = _run(inp, mode, mask)
        res = gate(got, rd[m], ex)
        say(f"  varlen{case} {mask} {mode}: {res.summary()}")
        assert res.ok, f"varlen{case} {mask} {mode}: {res.summary()}"
    assert np.array_equal(_run(inp, MODES[0], mask), _run(inp, MODES[0], mask)), "repeated launch changed the output"


@pytest.mark.parametrize("mask", ["none", "causal_br"])
def test_each_sequence_matches_the_fixed_length_entry_point(mask):
    lq, lk = (300, 64, 777), (500, 64, 777)
    wl = synth.VarlenWorkload("varlen_eq", lq, lk, 4, 2, MODES, mask=mask, seed=21)
    inp = synth.generate_varlen(wl)
    got = _run(inp, "rtna", mask)
    for b in range(wl.B):
        q0, q1, k0, k1 = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        q = to_device(np.ascontiguousarray(inp.q[q0:q1][None]))
        k = to_device(np.ascontiguousarray(inp.k[k0:k1][None]))
        v = to_device(np.ascontiguousarray(inp.v[k0:k1][None]))
        o = torch.empty_like(q)
        launch_gqa(q, k, v, o, "bshd", "rtna", mask)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(o)[0], got[q0:q1]), b


# Larger causal batches: grids of at least two rounds of 256 compute units (H=32 query heads over
# 8 K/V heads), sequences of odd and even q-tile counts (513, 1 and 256 rows have 3, 1 and 1),
# sequences without queries and without keys, bottom-right diagonals with Sk > Sq and Sk < Sq.
LARGE = [
    # (lengths_q, lengths_k, mask)
    ((1, 300, 0, 777, 1500, 513, 256), (1, 300, 0, 777, 1500, 513, 256), "causal"),
    ((1, 300, 0, 777, 1500, 513, 256), (5, 700, 10, 600, 1500, 2000, 0), "causal_br"),
]


def _grid(wl, max_q):
    n_qt = -(-max_q // 256)
    return 8 * -(-wl.B * wl.H_kv // 8) * (wl.H // wl.H_kv) * n_qt


@pytest.mark.parametrize("case", range(len(LARGE)))
def test_large_causal_varlen_all_rows(case):
    lq, lk, mask = LARGE[case]
    wl = synth.VarlenWorkload(f"varlen_large{case}", lq, lk, 32, 8, MODES, mask=mask, seed=41 + case)
    assert _grid(wl, max(lq)) >= 2 * 256, "the case must fill two rounds of compute units"
    inp = synth.generate_varlen(wl)
    ex, rd = oracle.attn_all_varlen(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, mask)
    for m, mode in enumerate(MODES):
        got = _run(inp, mode, mask)
        res = gate(got, rd[m], ex)
        say(f"  varlen_large{case} {mask} {mode}: {res.summary()}")
        assert res.ok, f"varlen_large{case} {mask} {mode}: {res.summary()}"
    # a larger max_seqlen_q only adds workgroups past every sequence's end
    assert np.array_equal(_run(inp, MODES[0], mask, max_q=3 * max(lq) + 7), _run(inp, MODES[0], mask))


@pytest.mark.parametrize("mask", ["causal", "causal_br"])
def test_large_causal_varlen_sequences_match_the_fixed_length_entry_point(mask):
    # each sequence alone through attn_fwd_bf16_gqa: the same arithmetic on the same rows, so the
    # same bits
    lq = (513, 64, 1025, 300)
    lk = lq if mask == "causal" else (700, 64, 1100, 1000)
    wl = synth.VarlenWorkload(f"varlen_large_eq_{mask}", lq, lk, 32, 8, MODES, mask=mask, seed=51)
    assert _grid(wl, max(lq)) >= 2 * 256
    inp = synth.generate_varlen(wl)
    got = _run(inp, "rtne", mask)
    for b in range(wl.B):
        q0, q1, k0, k1 = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        q = to_device(np.ascontiguousarray(inp.q[q0:q1][None]))
        k = to_device(np.ascontiguousarray(inp.k[k0:k1][None]))
        v = to_device(np.ascontiguousarray(inp.v[k0:k1][None]))
        o = torch.empty_like(q)
        launch_gqa(q, k, v, o, "bshd", "rtne", mask)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(o)[0], got[q0:q1]), b


def test_offsets_outside_the_tensors_are_clamped():
    # cu_seqlens past total_q / total_k (and a decreasing pair) are clamped on the
    # device: rows outside the tensors are never touched and sequence 0 stays right
    wl = synth.VarlenWorkload("varlen_bad", (40, 30), (50, 20), 2, 2, MODES, seed=31)
    inp = synth.generate_varlen(wl)
    ex, rd = oracle.attn_all_varlen(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    pad = torch.full((256, 2, 128), 1.0, dtype=torch.bfloat16, device="cuda:0")
    o_all = torch.cat([torch.zeros_like(q), pad]).contiguous()  # a sentinel block after o
    o = o_all[: q.shape[0]]
    cq = torch.tensor([0, 40, 1000], dtype=torch.int32, device="cuda:0")
    ck = torch.tensor([0, 50, -7], dtype=torch.int32, device="cuda:0")
    st = attn.attn_fwd_bf16_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), 0, cq.data_ptr(),
                                   ck.data_ptr(), 2, 2, 2, q.shape[0], k.shape[0], 1000, 0, 0,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o_all[q.shape[0]:], pad), "a row past the output tensor was written"
    res = gate(to_bits(o)[:40], rd[0][:40], ex[:40])
    assert res.ok, res.summary()
