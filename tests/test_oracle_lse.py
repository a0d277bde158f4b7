"""Pins for the oracle's per-row log-sum-exp, lse = log(sum_j exp(s_j)) over
the keys a row sees, with -Inf for a row that sees none (or only -Inf
logits) and NaN where the row's output is NaN.  The pages do not discuss it:
it is the per-row statistic the FlashAttention family keeps for a backward
pass or for merging key ranges (an extension beside grouped heads and packed batches).
Checked against exact logarithms of counts, numpy's logaddexp, scipy's and
torch's logsumexp on the same float64 logits, a dominant key, and the
special values.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from bf16_forward_attention_amd import synth
from tests import cases

D = 128


def lse_all(q, k, v, mask="none", layout="bhsd"):
    B, H, Sq, _ = q.shape
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(Sq)]
    _, _, lse = oracle.attn_rows(synth.to_layout(q, layout), synth.to_layout(k, layout), synth.to_layout(v, layout),
                                 layout, rows, mask=mask, with_lse=True)
    return lse.reshape(B, H, Sq)


def _random(B, H, Sq, Sk, seed, sigma=1.0, H_kv=None):
    return (cases.randn_bits((B, H, Sq, D), seed, sigma), cases.randn_bits((B, H_kv or H, Sk, D), seed + 1, sigma),
            cases.randn_bits((B, H_kv or H, Sk, D), seed + 2))


@pytest.mark.parametrize("mask", ["none", "causal", "causal_br"])
def test_uniform_logits_give_log_of_the_visible_count(mask):
    Sq, Sk = 9, 13
    q = np.zeros((1, 2, Sq, D), np.uint16)
    _, k, v = _random(1, 2, Sq, Sk, 3)
    lse = lse_all(q, k, v, mask)
    off = {"none": None, "causal": 0, "causal_br": Sk - Sq}[mask]
    for i in range(Sq):
        n = Sk if off is None else min(max(i + off + 1, 0), Sk)
        assert np.all(lse[0, :, i] == math.log(n)), (i, n)


@pytest.mark.parametrize("mask", ["none", "causal", "causal_br"])
@pytest.mark.parametrize("H_kv", [4, 2])
def test_matches_scipy_and_torch_logsumexp(mask, H_kv):
    B, H, Sq, Sk = 2, 4, 30, 77
    q, k, v = _random(B, H, Sq, Sk, 10, sigma=2.0, H_kv=H_kv)
    lse = lse_all(q, k, v, mask)
    s = np.einsum("bhid,bhjd->bhij", cases.val(q), np.repeat(cases.val(k), H // H_kv, axis=1)) / math.sqrt(128)
    if mask != "none":
        off = 0 if mask == "causal" else Sk - Sq
        s = np.where(np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] + off, s, -np.inf)
    ref = scipy.special.logsumexp(s, axis=-1)
    ref_t = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
    assert np.allclose(lse, ref, rtol=1e-14, atol=1e-13)
    assert np.allclose(lse, ref_t, rtol=1e-14, atol=1e-13)


@pytest.mark.parametrize("a", [-300.0, -2.0, 0.0, 3.5, 90.0])
def test_two_keys_follow_logaddexp(a):
    q = np.zeros((1, 1, 1, D), np.uint16)
    k = np.zeros((1, 1, 2, D), np.uint16)
    q[0, 0, 0, :8] = cases.bf(1.0)
    k[0, 0, 0, :8] = cases.bf(a)
    _, _, v = _random(1, 1, 1, 2, 20)
    lse = lse_all(q, k, v)
    assert lse[0, 0, 0] == pytest.approx(np.logaddexp(a * 8 / math.sqrt(128), 0.0), rel=1e-15, abs=1e-15)


def test_dominant_key_gives_its_logit_and_v_does_not_matter():
    q, k, v, jstar = cases.dominant(1, 2, 20, 50, seed=4)
    lse = lse_all(q, k, v)
    assert np.allclose(lse, 16384 / math.sqrt(128), rtol=2**-52, atol=0)
    _, _, v2 = _random(1, 2, 20, 50, 30)
    assert np.array_equal(lse_all(q, k, v2), lse)


def test_special_values():
    q, k, v = _random(1, 4, 6, 8, 40)
    k[0, 0, 3, 5] = 0x7FC0                        # NaN logit in every row of head 0
    k[0, 1, 2, 7] = 0x7F80                        # +Inf in head 1: rows with q[.,7] > 0 get +Inf
    q[0, 2, :, 0] = cases.bf(1.0)
    k[0, 2, :, 0] = 0xFF80                        # every logit of head 2 is -Inf
    lse = lse_all(q, k, v)
    assert np.all(np.isnan(lse[0, 0]))
    pos = cases.val(q[0, 1, :, 7]) > 0
    assert np.all(np.isnan(lse[0, 1][pos])) and np.all(np.isfinite(lse[0, 1][~pos]))
    assert np.all(lse[0, 2] == -np.inf)
    assert np.all(np.isfinite(lse[0, 3]))
    # bottom right with Sq > Sk: rows before the diagonal see no key
    q, k, v = _random(1, 1, 7, 3, 50)
    lse = lse_all(q, k, v, "causal_br")
    assert np.all(lse[0, 0, :4] == -np.inf) and np.all(np.isfinite(lse[0, 0, 4:]))


def test_varlen_rows_carry_their_sequence_lse():
    wl = synth.VarlenWorkload("t", (5, 7, 4), (9, 0, 6), 2, 1, ("rtne",), seed=6)
    inp = synth.generate_varlen(wl)
    rows = [(t, h) for t in range(16) for h in range(2)]
    _, _, lse = oracle.attn_rows_varlen(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, rows, with_lse=True)
    lse = lse.reshape(16, 2)
    assert np.all(lse[5:12] == -np.inf)
    _, _, l0 = oracle.attn_rows(inp.q[None, :5], inp.k[None, :9], inp.v[None, :9], "bshd",
                                [(0, h, i) for i in range(5) for h in range(2)], with_lse=True)
    assert np.array_equal(lse[:5].ravel(), l0)
