"""Pins for the oracle's grouped K/V heads (grouped-query attention).

The snilld.dk page "Open source attention kernel in HIP beats AITER v3 on
MI300X" lists GQA among what the kernel it describes leaves out (section
"Hvad er udgivet" / What was released) without defining it.  The reading
taken: K and V hold H_kv heads, H is a multiple of H_kv, and query head h
attends with K/V head h / (H / H_kv).  Checked against the already pinned
one-head-per-query-head oracle on K/V heads repeated group-wise (bit for bit,
with and without the causal masks), torch's float64 attention with
``enable_gqa``, and which query heads a change of one K/V head reaches.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from bf16_forward_attention_amd import synth
from tests import cases

MODES = ("rtne", "rtna", "rtz")
D = 128


def run_all(q, k, v, layout="bhsd", mask="none"):
    return oracle.attn_all(synth.to_layout(q, layout), synth.to_layout(k, layout), synth.to_layout(v, layout),
                           layout, mask=mask)


def _random(B, H, H_kv, Sq, Sk, seed, sigma=1.0):
    return (cases.randn_bits((B, H, Sq, D), seed, sigma), cases.randn_bits((B, H_kv, Sk, D), seed + 1, sigma),
            cases.randn_bits((B, H_kv, Sk, D), seed + 2))


@pytest.mark.parametrize("H,H_kv", [(8, 1), (8, 2), (8, 4), (6, 3), (4, 4)])
@pytest.mark.parametrize("mask", ["none", "causal", "causal_br"])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_equals_attention_on_repeated_kv_heads(H, H_kv, mask, layout):
    q, k, v = _random(2, H, H_kv, 19, 33, 10 + H + H_kv)
    ex, rd = run_all(q, k, v, layout, mask)
    g = H // H_kv
    ex_r, rd_r = run_all(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), layout, mask)
    assert np.array_equal(ex, ex_r, equal_nan=True) and np.array_equal(rd, rd_r)


@pytest.mark.parametrize("H,H_kv", [(8, 2), (12, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_float64_enable_gqa(H, H_kv, causal):
    q, k, v = _random(2, H, H_kv, 40, 200, 50)
    ex, rd = run_all(q, k, v, "bshd", "causal" if causal else "none")
    qt, kt, vt = (torch.from_numpy(cases.val(t)) for t in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, enable_gqa=True).numpy()
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    assert np.max(np.abs(ex - ref) / scale) < 1e-13
    for m, mode in enumerate(MODES):
        assert np.mean(oracle.round_bf16(ref, mode) == rd[m]) > 0.9999


def test_a_kv_head_reaches_exactly_its_query_heads():
    H, H_kv = 8, 2
    q, k, v = _random(1, H, H_kv, 10, 20, 70)
    ex1, _ = run_all(q, k, v)
    v2 = v.copy()
    v2[0, 1] = cases.randn_bits(v2[0, 1].shape, 71)  # K/V head 1 serves query heads 4..7
    ex2, _ = run_all(q, k, v2)
    changed = [not np.array_equal(ex1[0, h], ex2[0, h]) for h in range(H)]
    assert changed == [False] * 4 + [True] * 4


def test_head_counts_must_divide():
    q, k, v = _random(1, 6, 4, 3, 5, 80)
    with pytest.raises(ValueError):
        run_all(q, k, v)
