"""Pins for the oracle on variable-length batches (sequences packed one after
another, FlashAttention's "cu_seqlens" layout).

The snilld.dk page "Open source attention kernel in HIP beats AITER v3 on
MI300X" lists varlen batching among what the kernel it describes leaves out
and what serving with mixed lengths needs (sections "Hvad er udgivet" / What
was released and "Autoregressiv serving, de praktiske hager") without
defining it.  The reading: every sequence attends only within itself, as its
own fixed-length problem.  Checked against torch's float64 attention run per
sequence, a dominant key per sequence, and the sequences' independence.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
from bf16_forward_attention_amd import synth
from tests import cases

MODES = ("rtne", "rtna", "rtz")
D = 128


def _inputs(lq, lk, H=4, H_kv=2, seed=0, mask="none"):
    wl = synth.VarlenWorkload("t", tuple(lq), tuple(lk), H, H_kv, MODES, mask=mask, seed=seed)
    return synth.generate_varlen(wl)


@pytest.mark.parametrize("mask", ["none", "causal", "causal_br"])
def test_each_sequence_matches_torch_float64(mask):
    inp = _inputs([37, 1, 130, 64], [50, 9, 130, 200], seed=3, mask=mask)
    ex, rd = oracle.attn_all_varlen(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, mask)
    g = inp.wl.H // inp.wl.H_kv
    for b in range(inp.wl.B):
        q0, q1, k0, k1 = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        qt = torch.from_numpy(cases.val(inp.q[q0:q1])).transpose(0, 1)[None]  # [1, H, Sq, D]
        kt = torch.from_numpy(cases.val(inp.k[k0:k1])).transpose(0, 1)[None].repeat_interleave(g, 1)
        vt = torch.from_numpy(cases.val(inp.v[k0:k1])).transpose(0, 1)[None].repeat_interleave(g, 1)
        Sq, Sk = q1 - q0, k1 - k0
        attn_mask = None
        if mask == "causal":
            attn_mask = torch.ones(Sq, Sk, dtype=torch.bool).tril()
        elif mask == "causal_br":
            attn_mask = causal_lower_right(Sq, Sk)
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=attn_mask)[0].transpose(0, 1).numpy()
        got = ex[q0:q1]
        scale = np.max(np.abs(ref), axis=-1, keepdims=True)
        assert np.max(np.abs(got - ref) / scale) < 1e-13, b
        for m, mode in enumerate(MODES):
            assert np.mean(oracle.round_bf16(ref, mode) == rd[m, q0:q1]) > 0.999, (b, mode)


def test_dominant_key_stays_in_its_sequence():
    # in sequence b, every query row points along direction 1 + b and only key
    # j_b of that sequence has 128 there: each row returns V[j_b] of its own sequence
    lq, lk = [20, 33, 7, 64], [40, 5, 70, 64]
    inp = _inputs(lq, lk, H=2, H_kv=2, seed=5)
    q, k = np.zeros_like(inp.q), inp.k.copy()
    k[:, :, 1:5] = 0
    js = []
    for b in range(4):
        q[inp.cu_q[b]:inp.cu_q[b + 1], :, 1 + b] = cases.bf(128.0)
        j = inp.cu_k[b] + (7 * b + 3) % lk[b]
        k[j, :, 1 + b] = cases.bf(128.0)
        js.append(j)
    ex, rd = oracle.attn_all_varlen(q, k, inp.v, inp.cu_q, inp.cu_k)
    for b in range(4):
        for m in range(3):
            got = rd[m, inp.cu_q[b]:inp.cu_q[b + 1]]
            assert np.array_equal(got, np.broadcast_to(inp.v[js[b]], got.shape)), (b, m)


def test_sequences_are_independent_and_empty_keys_give_nan():
    inp = _inputs([10, 12, 6], [15, 0, 9], seed=7)
    ex, rd = oracle.attn_all_varlen(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k)
    assert np.all(np.isnan(ex[10:22])) and np.all(rd[:, 10:22] == 0x7FC0)
    assert np.all(np.isfinite(ex[:10])) and np.all(np.isfinite(ex[22:]))
    v2 = inp.v.copy()
    v2[15:] = cases.randn_bits(v2[15:].shape, 8)  # the keys of the third sequence
    ex2, _ = oracle.attn_all_varlen(inp.q, inp.k, v2, inp.cu_q, inp.cu_k)
    assert np.array_equal(ex2[:10], ex[:10]) and not np.array_equal(ex2[22:], ex[22:])


def test_one_sequence_is_the_fixed_length_problem():
    inp = _inputs([77], [130], H=4, H_kv=4, seed=9)
    ex, rd = oracle.attn_all_varlen(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, "causal_br")
    ex1, rd1 = oracle.attn_all(inp.q[None], inp.k[None], inp.v[None], "bshd", mask="causal_br")
    assert np.array_equal(ex, ex1[0].transpose(1, 0, 2)) and np.array_equal(rd, rd1[:, 0].transpose(0, 2, 1, 3))


def test_bad_offsets_are_rejected():
    inp = _inputs([3, 4], [5, 6], seed=1)
    with pytest.raises(ValueError):
        oracle.attn_all_varlen(inp.q, inp.k, inp.v, [0, 4, 3], inp.cu_k)
    with pytest.raises(ValueError):
        oracle.attn_all_varlen(inp.q, inp.k, inp.v, inp.cu_q, [0, 5, 12])
