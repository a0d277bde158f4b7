"""Pins for the oracle's attention: O = softmax(Q K^T / sqrt(128)) V.

The formula is the one the snilld.dk page states for the kernel (section
"Hvordan kernen arbejder" / How the kernel works); layouts BSHD/BHSD, d = 128
and unequal lengths come from its section "Hvad er udgivet" (What was
released).  Each test below checks the oracle against something other than
its own formula: a closed form, an invariant of the mathematics, a library
routine (scipy's logistic function, torch's float64 softmax), or brute force
at 50 significant digits on tiny inputs.
"""
import math
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from bf16_forward_attention_amd import synth
from tests import cases
from tests.bf16_exact import round_exact, tie_distance

MODES = ("rtne", "rtna", "rtz")
D = 128


def run_all(q, k, v, layout="bhsd"):
    """Oracle on logical inputs stored in ``layout``; logical-order outputs."""
    return oracle.attn_all(synth.to_layout(q, layout), synth.to_layout(k, layout), synth.to_layout(v, layout), layout)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("Sk", [1, 2, 3, 7, 100])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_uniform_logits_give_mean_of_v(Sk, layout):
    # Q = 0 makes every logit 0, so every weight is 1/Sk: O = (sum_j V_j) / Sk
    B, H, Sq = 1, 2, 3
    q = np.zeros((B, H, Sq, D), np.uint16)
    k = cases.randn_bits((B, H, Sk, D), 5)
    v = cases.randn_bits((B, H, Sk, D), 6)
    ex, rd = run_all(q, k, v, layout)
    vals = cases.val(v)
    checked = 0
    for b in range(B):
        for h in range(H):
            for c in range(D):
                exact = sum(Fraction(float(x)) for x in vals[b, h, :, c]) / Sk
                near = tie_distance(exact)
                if 0 < near < Fraction(1, 2**40):
                    continue  # binary64 cannot decide this one; both neighbours are right
                for m, mode in enumerate(MODES):
                    want = round_exact(exact, mode)
                    for i in range(Sq):
                        assert int(rd[m, b, h, i, c]) == want
                checked += 1
    assert checked > 0.99 * B * H * D


@pytest.mark.parametrize("shape", [(1, 1, 5, 9), (2, 3, 130, 67), (1, 2, 64, 129)])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_dominant_logit_returns_that_v_row(shape, layout):
    B, H, Sq, Sk = shape
    q, k, v, jstar = cases.dominant(B, H, Sq, Sk, seed=3)
    _, rd = run_all(q, k, v, layout)
    for m in range(3):
        for b in range(B):
            for h in range(H):
                assert np.array_equal(rd[m, b, h], v[b, h, jstar[b, h]])


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_single_key_returns_v0(layout):
    q = cases.randn_bits((2, 3, 17, D), 8, sigma=3.0)
    k = cases.randn_bits((2, 3, 1, D), 9, sigma=3.0)
    v = cases.randn_bits((2, 3, 1, D), 10)
    _, rd = run_all(q, k, v, layout)
    for m in range(3):
        assert np.array_equal(rd[m], np.broadcast_to(v, (2, 3, 17, D)))


@pytest.mark.parametrize("a", [-100.0, -3.0, -0.5, 0.0, 0.25, 2.0, 40.0, 88.0])
def test_two_keys_follow_the_logistic_function(a):
    # keys with logits s0 = a * 8 / sqrt(128) and s1 = 0: the weight of key 0 is
    # the logistic function of s0 - s1 (softmax of two entries)
    q = np.zeros((1, 1, 1, D), np.uint16)
    k = np.zeros((1, 1, 2, D), np.uint16)
    v = np.zeros((1, 1, 2, D), np.uint16)
    q[0, 0, 0, :8] = cases.bf(1.0)
    k[0, 0, 0, :8] = cases.bf(a)
    v[0, 0, 0, 0] = cases.bf(1.0)  # column 0 reads the weight of key 0
    v[0, 0, 1, 1] = cases.bf(1.0)  # column 1 reads the weight of key 1
    ex, _ = run_all(q, k, v)
    s0 = a * 8 / math.sqrt(128)
    assert ex[0, 0, 0, 0] == pytest.approx(scipy.special.expit(s0), rel=4e-16, abs=1e-300)
    assert ex[0, 0, 0, 1] == pytest.approx(scipy.special.expit(-s0), rel=4e-16, abs=1e-300)
    assert np.all(ex[0, 0, 0, 2:] == 0.0)


@pytest.mark.parametrize("row", range(len(cases.load_ties())))
def test_midpoint_ties_golden(row):
    vals, want, _scope = cases.load_ties()[row]
    q, k, v = cases.tie_inputs(vals)
    _, rd = run_all(q, k, v)
    for m in range(3):
        assert np.all(rd[m, 0, 0, 0] == want[m]), (vals, MODES[m])


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def _random(B, H, Sq, Sk, seed, sigma=1.0):
    return (cases.randn_bits((B, H, Sq, D), seed, sigma), cases.randn_bits((B, H, Sk, D), seed + 1, sigma),
            cases.randn_bits((B, H, Sk, D), seed + 2))


def test_negating_v_negates_o_bit_exactly():
    q, k, v = _random(1, 2, 20, 45, 20)
    _, a = run_all(q, k, v)
    _, b = run_all(q, k, v ^ np.uint16(0x8000))
    assert np.array_equal(a ^ np.uint16(0x8000), b)


def test_scaling_v_by_power_of_two_scales_o():
    q, k, v = _random(1, 2, 20, 45, 30)
    _, a = run_all(q, k, v)
    v4 = cases.bf(cases.val(v) * 4.0)
    _, b = run_all(q, k, v4)
    assert np.array_equal(cases.val(b), cases.val(a) * 4.0)


def test_layouts_agree_bit_exactly():
    q, k, v = _random(2, 3, 33, 70, 40)
    ex1, r1 = run_all(q, k, v, "bshd")
    ex2, r2 = run_all(q, k, v, "bhsd")
    assert np.array_equal(ex1, ex2) and np.array_equal(r1, r2)


def test_other_heads_do_not_leak():
    q, k, v = _random(2, 3, 16, 40, 50)
    ex1, _ = run_all(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[1, 2] = cases.randn_bits(k2[1, 2].shape, 99)
    v2[0, 1] = cases.randn_bits(v2[0, 1].shape, 98)
    ex2, _ = run_all(q, k2, v2)
    same = np.ones((2, 3), bool)
    same[1, 2] = same[0, 1] = False
    for b in range(2):
        for h in range(3):
            assert np.array_equal(ex1[b, h], ex2[b, h]) == bool(same[b, h])


def test_permuting_keys_leaves_o_unchanged():
    q, k, v = _random(1, 2, 24, 90, 60)
    perm = np.random.default_rng(1).permutation(90)
    ex1, r1 = run_all(q, k, v)
    ex2, r2 = run_all(q, k[:, :, perm], v[:, :, perm])
    scale = np.max(np.abs(ex1), axis=-1, keepdims=True)
    assert np.all(np.abs(ex1 - ex2) <= 1e-13 * scale)
    # rounded outputs agree except where the exact value sits on a rounding boundary
    assert np.mean(r1 == r2) > 0.9999


def test_softmax_rows_sum_to_one():
    q, k, _ = _random(1, 2, 4, 333, 70, sigma=2.0)
    qs, ks = synth.to_layout(q, "bshd"), synth.to_layout(k, "bshd")
    for h in range(2):
        for i in range(4):
            w, l = oracle.softmax_row(qs, ks, "bshd", 0, h, i)
            assert l >= 1.0  # the maximal key contributes exp(0) = 1
            assert abs(math.fsum(w) - 1.0) <= 333 * 2.0**-52
            assert np.all(w >= 0) and np.isclose(w.max(), 1.0 / l, rtol=0, atol=1e-16)


# --------------------------------------------------------------------------
# NaN / Inf propagation (IEEE evaluation of the max-subtracted formula)
# --------------------------------------------------------------------------
def test_nan_in_k_poisons_its_whole_head():
    q, k, v = _random(1, 3, 10, 20, 80)
    k[0, 1, 7, 33] = 0x7FC0
    ex, rd = run_all(q, k, v)
    assert np.all(np.isnan(ex[0, 1])) and not np.any(np.isnan(ex[0, [0, 2]]))
    assert np.all(rd[:, 0, 1] == 0x7FC0)


def test_nan_in_q_poisons_its_row():
    q, k, v = _random(1, 2, 10, 20, 90)
    q[0, 0, 4, 100] = 0xFFC1
    ex, _ = run_all(q, k, v)
    nan_rows = np.all(np.isnan(ex), axis=-1)
    assert nan_rows[0, 0, 4] and nan_rows.sum() == 1 and not np.any(np.isnan(ex[~nan_rows]))


@pytest.mark.parametrize("inf_bits", [0x7F80, 0xFF80])
def test_inf_in_k_nan_rows_follow_sign_and_other_rows_drop_the_key(inf_bits):
    # k[j*, c*] = +-Inf: rows with q[c*] of the same sign get a +Inf logit -> NaN row;
    # rows with the opposite sign get a -Inf logit -> key j* has weight 0 exactly
    B, H, Sq, Sk = 1, 1, 40, 30
    q, k, v = _random(B, H, Sq, Sk, 100)
    js, cs = 11, 57
    k[0, 0, js, cs] = inf_bits
    q[0, 0, 5, cs] = 0  # 0 * Inf = NaN: NaN row whatever the sign
    ex, rd = run_all(q, k, v)
    keep = [j for j in range(Sk) if j != js]
    ex_drop, rd_drop = run_all(q, k[:, :, keep], v[:, :, keep])
    qsign = np.sign(cases.val(q[0, 0, :, cs]))
    isign = 1.0 if inf_bits == 0x7F80 else -1.0
    for i in range(Sq):
        if qsign[i] * isign > 0 or qsign[i] == 0:
            assert np.all(np.isnan(ex[0, 0, i])), i
        else:
            assert np.array_equal(ex[0, 0, i], ex_drop[0, 0, i]), i
            assert np.array_equal(rd[:, 0, 0, i], rd_drop[:, 0, 0, i]), i
    assert np.any(qsign * isign > 0) and np.any(qsign * isign < 0)


def test_all_logits_minus_inf_give_nan_row():
    q, k, v = _random(1, 1, 3, 6, 110)
    q[0, 0, :, 0] = cases.bf(1.0)
    k[0, 0, :, 0] = 0xFF80  # every logit of every row is -Inf
    ex, _ = run_all(q, k, v)
    assert np.all(np.isnan(ex))


def test_inf_in_v_only_touches_its_column():
    q, k, v = _random(1, 1, 5, 9, 120)
    v[0, 0, 4, 10] = 0x7F80
    ex, rd = run_all(q, k, v)
    assert np.all(np.isposinf(ex[0, 0, :, 10]))
    others = np.delete(ex[0, 0], 10, axis=1)
    assert np.all(np.isfinite(others))


def test_nan_inf_rules_agree_with_torch_softmax():
    # library cross-check of the NaN rows: torch float64 softmax of the same logits
    q, k, v = _random(1, 2, 12, 16, 130)
    k[0, 0, 3, 9] = 0x7F80
    k[0, 1, 5, 2] = 0xFF80
    q[0, 1, 0, :] = 0
    q[0, 1, 0, 2] = cases.bf(1.0)
    ex, _ = run_all(q, k, v)
    with np.errstate(invalid="ignore"):
        qt, kt, vt = (torch.from_numpy(cases.val(t)) for t in (q, k, v))
        ref = torch.softmax(qt @ kt.transpose(-1, -2).contiguous() / math.sqrt(128), dim=-1) @ vt
    assert np.array_equal(np.isnan(ex), np.isnan(ref.numpy()))


# --------------------------------------------------------------------------
# brute force and library cross-checks
# --------------------------------------------------------------------------
def test_brute_force_mpmath_tiny():
    mpmath.mp.dps = 50
    rng_seed = 140
    B, H, Sq, Sk = 1, 2, 3, 6
    q, k, v = _random(B, H, Sq, Sk, rng_seed, sigma=1.5)
    _, rd = run_all(q, k, v)
    qv, kv, vv = cases.val(q), cases.val(k), cases.val(v)
    flagged = 0
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                s = [mpmath.fsum(mpmath.mpf(float(qv[b, h, i, c])) * mpmath.mpf(float(kv[b, h, j, c]))
                                 for c in range(D)) / mpmath.sqrt(128) for j in range(Sk)]
                m = max(s)
                w = [mpmath.exp(x - m) for x in s]
                l = mpmath.fsum(w)
                for c in range(D):
                    o = mpmath.fsum(w[j] * mpmath.mpf(float(vv[b, h, j, c])) for j in range(Sk)) / l
                    exact = Fraction(mpmath.nstr(o, 45, min_fixed=-10**9, max_fixed=10**9))
                    if tie_distance(exact) < Fraction(1, 10**12):
                        flagged += 1
                        continue
                    for mi, mode in enumerate(MODES):
                        assert int(rd[mi, b, h, i, c]) == round_exact(exact, mode), (b, h, i, c, mode)
    assert flagged <= 2


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_matches_torch_float64_softmax(layout):
    B, H, Sq, Sk = 2, 3, 37, 300
    q, k, v = _random(B, H, Sq, Sk, 150, sigma=1.0)
    ex, rd = run_all(q, k, v, layout)
    qt, kt, vt = (torch.from_numpy(cases.val(t)) for t in (q, k, v))
    ref = (torch.softmax(qt @ kt.transpose(-1, -2).contiguous() / math.sqrt(128), dim=-1) @ vt).numpy()
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    assert np.max(np.abs(ex - ref) / scale) < 1e-13
    for m, mode in enumerate(MODES):
        from_ref = oracle.round_bf16(ref, mode)
        assert np.mean(from_ref == rd[m]) > 0.9999
