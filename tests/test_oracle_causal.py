"""Pins for the oracle's causal mask.

The snilld.dk page "Open source attention kernel in HIP beats AITER v3 on
MI300X" names the causal mask as missing from the kernel it describes and as
what autoregressive serving needs (sections "Hvad er udgivet" / What was
released and "Autoregressiv serving, de praktiske hager"); it gives no
definition.  The reading taken: query row i attends to the keys
j <= i + off, with off = 0 ("causal", diagonal at the top left) or
off = Sk - Sq ("causal_br", diagonal at the bottom right); masked keys take no
part, and a row with no visible key is NaN (0/0).  Each test checks the oracle
against something other than its own formula: exact rational means, a
dominant key on the diagonal, the already pinned unmasked oracle on the
visible keys, perturbations past the diagonal, mpmath at 50 digits, and
torch's float64 attention with its own causal masks.
"""
import math
import warnings
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
from bf16_forward_attention_amd import synth
from tests import cases
from tests.bf16_exact import round_exact, tie_distance

MODES = ("rtne", "rtna", "rtz")
D = 128
SHAPES = [(7, 7), (5, 12), (12, 5), (1, 9), (9, 1)]  # (Sq, Sk)


def run_all(q, k, v, mask, layout="bhsd"):
    return oracle.attn_all(synth.to_layout(q, layout), synth.to_layout(k, layout), synth.to_layout(v, layout),
                           layout, mask=mask)


def visible(mask, i, Sq, Sk):
    """Keys row i sees, written out from the reading (not the oracle's code)."""
    if mask == "causal":
        return [j for j in range(Sk) if j <= i]
    return [j for j in range(Sk) if j - (Sk - Sq) <= i]


def _random(B, H, Sq, Sk, seed, sigma=1.0):
    return (cases.randn_bits((B, H, Sq, D), seed, sigma), cases.randn_bits((B, H, Sk, D), seed + 1, sigma),
            cases.randn_bits((B, H, Sk, D), seed + 2))


@pytest.mark.parametrize("mask", ["causal", "causal_br"])
@pytest.mark.parametrize("shape", SHAPES)
def test_uniform_logits_give_mean_of_visible_v(mask, shape):
    # Q = 0: every logit is 0, so row i is the exact mean of its visible V rows
    Sq, Sk = shape
    q = np.zeros((1, 1, Sq, D), np.uint16)
    k = cases.randn_bits((1, 1, Sk, D), 11)
    v = cases.randn_bits((1, 1, Sk, D), 12)
    ex, rd = run_all(q, k, v, mask)
    vals = cases.val(v)[0, 0]
    for i in range(Sq):
        vis = visible(mask, i, Sq, Sk)
        if not vis:
            assert np.all(np.isnan(ex[0, 0, i])) and np.all(rd[:, 0, 0, i] == 0x7FC0)
            continue
        for c in range(D):
            exact = sum(Fraction(float(vals[j, c])) for j in vis) / len(vis)
            if 0 < tie_distance(exact) < Fraction(1, 2**40):
                continue
            for m, mode in enumerate(MODES):
                assert int(rd[m, 0, 0, i, c]) == round_exact(exact, mode), (i, c, mode)


@pytest.mark.parametrize("mask", ["causal", "causal_br"])
@pytest.mark.parametrize("shape", [(6, 6), (4, 10), (10, 4)])
def test_dominant_key_on_the_diagonal(mask, shape):
    # q_i and k_j point along direction 1 + (j mod 127); row i's last visible key
    # j = i + off has logit ~1448 against 0 for every other key it sees, so
    # O_i = V_j exactly in every mode
    Sq, Sk = shape
    off = 0 if mask == "causal" else Sk - Sq
    q = np.zeros((1, 1, Sq, D), np.uint16)
    k = np.zeros((1, 1, Sk, D), np.uint16)
    v = cases.randn_bits((1, 1, Sk, D), 21)
    for j in range(Sk):
        k[0, 0, j, 1 + j % 127] = cases.bf(128.0)
    for i in range(Sq):
        j = i + off
        if 0 <= j < Sk:
            q[0, 0, i, 1 + j % 127] = cases.bf(128.0)
    ex, rd = run_all(q, k, v, mask)
    for i in range(Sq):
        j = min(i + off, Sk - 1)
        if j < 0:
            assert np.all(np.isnan(ex[0, 0, i]))
        elif i + off < Sk:
            for m in range(3):
                assert np.array_equal(rd[m, 0, 0, i], v[0, 0, j]), (i, j)


@pytest.mark.parametrize("mask", ["causal", "causal_br"])
@pytest.mark.parametrize("shape", SHAPES)
def test_row_equals_unmasked_attention_on_its_visible_keys(mask, shape):
    Sq, Sk = shape
    q, k, v = _random(1, 2, Sq, Sk, 30, sigma=1.5)
    ex, rd = run_all(q, k, v, mask)
    for i in range(Sq):
        vis = visible(mask, i, Sq, Sk)
        if not vis:
            assert np.all(np.isnan(ex[:, :, i]))
            continue
        n = len(vis)
        assert vis == list(range(n))
        ex_u, rd_u = run_all(q[:, :, i:i + 1], k[:, :, :n].copy(), v[:, :, :n].copy(), "none")
        assert np.array_equal(ex[:, :, i], ex_u[:, :, 0]), i
        assert np.array_equal(rd[:, :, :, i], rd_u[:, :, :, 0]), i


@pytest.mark.parametrize("mask", ["causal", "causal_br"])
def test_keys_past_the_diagonal_do_not_matter(mask):
    Sq, Sk = 9, 14
    q, k, v = _random(1, 1, Sq, Sk, 40)
    ex1, _ = run_all(q, k, v, mask)
    cut = 6  # keys >= 6 replaced
    k2, v2 = k.copy(), v.copy()
    k2[:, :, cut:] = cases.randn_bits(k2[:, :, cut:].shape, 41, 3.0)
    v2[:, :, cut:] = cases.randn_bits(v2[:, :, cut:].shape, 42)
    ex2, _ = run_all(q, k2, v2, mask)
    for i in range(Sq):
        sees_changed = max(visible(mask, i, Sq, Sk), default=-1) >= cut
        assert np.array_equal(ex1[0, 0, i], ex2[0, 0, i]) != sees_changed, i


def test_bottom_right_rows_before_the_diagonal_are_nan():
    Sq, Sk = 10, 4
    q, k, v = _random(2, 2, Sq, Sk, 50)
    ex, rd = run_all(q, k, v, "causal_br")
    nan_rows = np.all(np.isnan(ex), axis=-1)
    assert np.array_equal(nan_rows, np.broadcast_to(np.arange(Sq) < Sq - Sk, nan_rows.shape))
    assert np.all(rd[:, nan_rows] == 0x7FC0)
    assert np.all(np.isfinite(ex[~nan_rows]))


def test_square_masks_coincide_and_differ_from_none():
    q, k, v = _random(1, 2, 11, 11, 60)
    a = run_all(q, k, v, "causal")
    b = run_all(q, k, v, "causal_br")
    n = run_all(q, k, v, "none")
    assert np.array_equal(a[1], b[1])
    assert np.array_equal(a[1][:, :, :, -1], n[1][:, :, :, -1])  # the last row sees every key
    assert not np.array_equal(a[1][:, :, :, 0], n[1][:, :, :, 0])


@pytest.mark.parametrize("mask", ["causal", "causal_br"])
@pytest.mark.parametrize("shape", [(37, 300), (300, 37), (64, 64)])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_matches_torch_float64_causal_attention(mask, shape, layout):
    Sq, Sk = shape
    q, k, v = _random(2, 2, Sq, Sk, 70)
    ex, rd = run_all(q, k, v, mask, layout)
    qt, kt, vt = (torch.from_numpy(cases.val(t)) for t in (q, k, v))
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")  # torch warns that lower-right rows with no key are undefined
        if mask == "causal":
            ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
        else:
            ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=causal_lower_right(Sq, Sk))
    ref = ref.numpy()
    rows = np.array([bool(visible(mask, i, Sq, Sk)) for i in range(Sq)])
    assert rows.any()
    ex, ref, rd = ex[:, :, rows], ref[:, :, rows], rd[:, :, :, rows]
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    assert np.max(np.abs(ex - ref) / scale) < 1e-13
    for m, mode in enumerate(MODES):
        assert np.mean(oracle.round_bf16(ref, mode) == rd[m]) > 0.9999


@pytest.mark.parametrize("mask", ["causal", "causal_br"])
def test_brute_force_mpmath_tiny(mask):
    mpmath.mp.dps = 50
    Sq, Sk = 4, 6
    q, k, v = _random(1, 1, Sq, Sk, 80, sigma=1.5)
    _, rd = run_all(q, k, v, mask)
    qv, kv, vv = cases.val(q)[0, 0], cases.val(k)[0, 0], cases.val(v)[0, 0]
    flagged = 0
    for i in range(Sq):
        vis = visible(mask, i, Sq, Sk)
        s = [mpmath.fsum(mpmath.mpf(float(qv[i, c])) * mpmath.mpf(float(kv[j, c])) for c in range(D))
             / mpmath.sqrt(128) for j in vis]
        mx = max(s)
        w = [mpmath.exp(x - mx) for x in s]
        l = mpmath.fsum(w)
        for c in range(D):
            o = mpmath.fsum(wj * mpmath.mpf(float(vv[j, c])) for wj, j in zip(w, vis)) / l
            exact = Fraction(mpmath.nstr(o, 45, min_fixed=-10**9, max_fixed=10**9))
            if tie_distance(exact) < Fraction(1, 10**12):
                flagged += 1
                continue
            for m, mode in enumerate(MODES):
                assert int(rd[m, 0, 0, i, c]) == round_exact(exact, mode), (i, c, mode)
    assert flagged <= 2


def test_unknown_mask_is_rejected():
    q, k, v = _random(1, 1, 2, 2, 90)
    with pytest.raises(ValueError):
        run_all(q, k, v, "upper")
    assert math.isfinite(float(run_all(q, k, v, "causal")[0][0, 0, 1, 0]))
