"""GPU parity on bf16 subnormal inputs and outputs.

The oracle decodes and rounds subnormals exactly (gradual underflow); the
kernel runs with fp32 denormals preserved (kernel descriptor denorm mode 3), so
subnormal V values, subnormal Q or K elements and outputs whose whole row is
subnormal must come out as the oracle says: bit for bit where the exact
result is reachable in fp32 without rounding, within the row-scaled 2-ULP gate
otherwise (at a subnormal row scale that is two subnormal steps, 2 * 2^-133,
so a row flushed to zero fails it).  The snilld.dk page asks that every bf16
output stay within the stated ULP bound of the reference (section "Numerik
samlet et sted" / Numerics in one place); subnormals are part of bf16.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import cases
from tests.gate import gate
from tests.gpu_util import MODES, run_logical, say

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


def _logical_oracle(q, k, v, mask="none"):
    """Oracle on logical [B, H, S, 128] arrays (stored as BHSD, which is the logical order)."""
    return oracle.attn_all(np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v), "bhsd",
                           mask=mask)


def _is_subnormal(bits):
    b = np.asarray(bits)
    return ((b & 0x7F80) == 0) & ((b & 0x7F) != 0)


def test_single_key_subnormal_v_exact():
    # one key: the weight is 1 and O = V_0 in every mode; V_0 spans the subnormal significands 1..127, both signs
    v0 = np.concatenate([np.arange(1, 128, 2, dtype=np.uint16), np.arange(1, 128, 2, dtype=np.uint16) | 0x8000])
    v = np.broadcast_to(v0, (1, 2, 1, D)).copy()
    q = cases.randn_bits((1, 2, 70, D), 40, sigma=3.0)
    k = cases.randn_bits((1, 2, 1, D), 41, sigma=3.0)
    ex, rd = _logical_oracle(q, k, v)
    for m, mode in enumerate(MODES):
        assert np.array_equal(rd[m], np.broadcast_to(v, rd[m].shape)), "oracle: one key must give V_0"
        for layout in ("bshd", "bhsd"):
            got = run_logical(q, k, v, layout, mode)
            assert np.array_equal(got, np.broadcast_to(v, got.shape)), (mode, layout)


@pytest.mark.parametrize("Sk", [64 * 3 + 3, 64 * 2 + 63, 200])
def test_dominant_key_subnormal_v_exact(Sk):
    # a dominant key (other weights underflow to exactly 0) returns its subnormal V row bit for bit,
    # including when that key sits in the ragged last key tile
    q, k, _, jstar = cases.dominant(1, 2, 130, Sk, seed=Sk)
    v = cases.subnormal_bits((1, 2, Sk, D), seed=Sk)
    for mode in MODES:
        got = run_logical(q, k, v, "bhsd", mode)
        for h in range(2):
            assert np.array_equal(got[0, h], v[0, h, jstar[0, h]]), (mode, h)


@pytest.mark.parametrize("n", [2, 64, 192, 1024])
def test_uniform_logits_subnormal_v_mean(n):
    # Q = 0: every weight is exactly 1, so O is the mean of n subnormal V rows.  With n a power of two
    # every partial sum, 1/n and the quotient are exact in fp32 (multiples of 2^-149), so the GPU's
    # bits must equal the oracle's exact rounding in every mode; n = 192 (not a power of two) is held
    # to the gate.
    q = np.zeros((1, 2, 33, D), np.uint16)
    k = cases.randn_bits((1, 2, n, D), 50 + n)
    v = cases.subnormal_bits((1, 2, n, D), seed=60 + n)
    ex, rd = _logical_oracle(q, k, v)
    exact = n & (n - 1) == 0
    for m, mode in enumerate(MODES):
        got = run_logical(q, k, v, "bhsd", mode)
        res = gate(got, rd[m], ex)
        say(f"  n={n} {mode}: {res.summary()} subnormal outputs {int(_is_subnormal(got).sum())}")
        assert _is_subnormal(rd[m]).any()
        assert res.ok, (mode, res.summary())
        if exact:
            assert np.array_equal(got, rd[m]), (mode, np.argwhere(got != rd[m])[:4].tolist())


def test_midpoint_of_the_two_smallest_subnormals():
    # V values 2^-133 and 2^-132 under equal logits: the mean 1.5 * 2^-133 is the midpoint of the
    # two smallest subnormals, exact in fp32; RTNE 0x0002, RTNA 0x0002, RTZ 0x0001
    q, k, v = cases.tie_inputs([0x0001, 0x0002])
    want = (0x0002, 0x0002, 0x0001)
    q2, k2, v2 = cases.tie_inputs([0x8001, 0x8002])
    for m, mode in enumerate(MODES):
        assert np.all(run_logical(q, k, v, "bhsd", mode) == want[m]), mode
        assert np.all(run_logical(q2, k2, v2, "bhsd", mode) == (want[m] | 0x8000)), mode


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_rows_with_subnormal_output(layout):
    # random logits over subnormal V: every output row is subnormal, so the gate's tolerance is two
    # subnormal steps and a flush to zero anywhere in the products or the rescale would fail it
    q = cases.randn_bits((2, 2, 150, D), 70)
    k = cases.randn_bits((2, 2, 333, D), 71)
    v = cases.subnormal_bits((2, 2, 333, D), seed=72)
    ex, rd = _logical_oracle(q, k, v)
    assert np.all(np.abs(ex) < 2.0**-126)
    for m, mode in enumerate(MODES):
        got = run_logical(q, k, v, layout, mode)
        res = gate(got, rd[m], ex)
        say(f"  {layout} {mode}: {res.summary()}")
        assert res.ok, (mode, res.summary())
        assert np.count_nonzero(got) > 0.9 * got.size


@pytest.mark.parametrize("which", ["q", "k"])
def test_subnormal_q_or_k_elements_carry_normal_logits(which):
    # Dims 0..31 of Q (or K) hold subnormals and the same dims of the other operand hold values near
    # 2^126, so each of those products is of order one: the logits (and so the weights) depend on the
    # subnormal elements as much as on dims 32..127, which are N(0,1) on both sides.  A kernel that
    # flushed subnormal MFMA inputs to zero would drop half of every logit and fail the gate.
    B, H, Sq, Sk = 1, 2, 130, 300
    q = cases.randn_bits((B, H, Sq, D), 80)
    k = cases.randn_bits((B, H, Sk, D), 81)
    small, big = (q, k) if which == "q" else (k, q)
    n_small = small.shape[2]
    small[..., :32] = cases.subnormal_bits((B, H, n_small, 32), seed=82)
    big[..., :32] = cases.scaled_bits(big[..., :32].shape, seed=83, exp_shift=126)
    v = cases.randn_bits((B, H, Sk, D), 84)
    ex, rd = _logical_oracle(q, k, v)
    # the subnormal part of the logits is not negligible: zeroing it changes the exact output
    zeroed = small.copy()
    zeroed[..., :32] = 0
    ex0, _ = _logical_oracle(zeroed, k, v) if which == "q" else _logical_oracle(q, zeroed, v)
    assert np.max(np.abs(ex0 - ex)) > 0.05
    for m, mode in enumerate(MODES):
        got = run_logical(q, k, v, "bshd", mode)
        res = gate(got, rd[m], ex)
        say(f"  subnormal {which} {mode}: {res.summary()}")
        assert res.ok, (mode, res.summary())
