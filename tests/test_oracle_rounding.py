"""Pins for the oracle's bf16 decoding and its three output roundings.

The modes are the three the pages benchmark (RTNE, RTNA, RTZ: tilnote.io
page, section on the performance figures; snilld.dk page, section on
numerics), read as IEEE-754 roundTiesToEven, roundTiesToAway and
roundTowardZero.  Nothing here re-runs the oracle's own procedure: each
check uses a closed form, a library routine or a definitional search.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from tests.bf16_exact import round_exact

MODES = ("rtne", "rtna", "rtz")


def _f32_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def test_decode_exhaustive_matches_float32_extension():
    # closed form: a bf16 pattern is the top half of the float32 with the same value
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_bf16(bits)
    want = _f32_bits_to_f64(bits.astype(np.uint32) << np.uint32(16))
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, got[0x8000]) == -1.0 and got[0x8000] == 0.0


def _structured_f32_patterns() -> np.ndarray:
    """Every bf16 high half combined with low halves at and around the ties."""
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    rng = np.random.default_rng(1)
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFE, 0xFFFF]
                    + list(rng.integers(0, 1 << 16, 6)), dtype=np.uint32)
    return (hi[:, None] | lows[None, :]).ravel()


def test_round_float32_inputs_closed_forms():
    bits = _structured_f32_patterns()
    x = _f32_bits_to_f64(bits)
    nan = np.isnan(x)
    top = (bits >> np.uint32(16)).astype(np.uint16)

    # RTZ of a float32 is its top 16 bits (truncation of the significand)
    rtz = oracle.round_bf16(x, "rtz")
    assert np.array_equal(rtz[~nan], top[~nan])

    # RTNA of a float32: add half an ulp of bf16 to the magnitude bits, truncate
    rtna = oracle.round_bf16(x, "rtna")
    want = ((bits + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(rtna[~nan], want[~nan])

    # every NaN becomes the canonical quiet NaN
    for mode in MODES:
        assert np.all(oracle.round_bf16(x[nan], mode) == 0x7FC0)


def test_round_float32_inputs_rtne_matches_torch():
    # library routine: PyTorch's CPU float32 -> bfloat16 conversion rounds to nearest even
    bits = _structured_f32_patterns()
    x = _f32_bits_to_f64(bits)
    nan = np.isnan(x)
    got = oracle.round_bf16(x, "rtne")
    ref = torch.from_numpy(bits.view(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("mode", MODES)
def test_round_random_float64_definitional(mode):
    # binary64 inputs that are not float32 values: bisection over all bf16 values
    rng = np.random.default_rng(7)
    xs = np.concatenate([
        rng.standard_normal(400) * np.exp2(rng.integers(-140, 130, 400)),
        rng.standard_normal(200),
        np.exp2(rng.uniform(-135, -120, 100)),  # bf16 subnormal range
        np.exp2(rng.uniform(126, 129, 50)) * rng.choice([-1, 1], 50),  # overflow edge
    ])
    got = oracle.round_bf16(xs, mode)
    for x, g in zip(xs, got):
        assert int(g) == round_exact(float(x), mode), (x, mode)


@pytest.mark.parametrize("mode", MODES)
def test_round_exact_ties_and_near_ties(mode):
    # midpoints between neighbouring bf16 values, and one binary64 ulp either side
    rng = np.random.default_rng(11)
    pats = np.concatenate([rng.integers(0, 0x7F7F, 300), [0, 1, 0x7E, 0x7F, 0x80, 0x3F80, 0x7F7E]])
    for p in pats:
        lo = Fraction(float(np.array([int(p) << 16], dtype=np.uint32).view(np.float32)[0]))
        hi = Fraction(float(np.array([(int(p) + 1) << 16], dtype=np.uint32).view(np.float32)[0]))
        mid = float((lo + hi) / 2)  # exact in binary64
        for x in (mid, math.nextafter(mid, 0.0), math.nextafter(mid, math.inf)):
            for s in (1.0, -1.0):
                assert int(oracle.round_bf16(np.array([s * x]), mode)[0]) == round_exact(s * x, mode)


def test_round_specials_and_overflow():
    bmax = float(np.array([0x7F7F << 16], dtype=np.uint32).view(np.float32)[0])
    ulp_max = 2.0 ** (127 - 7)
    cases = [  # (x, (rtne, rtna, rtz)); a list, since 0.0 == -0.0 as dict keys
        (0.0, (0x0000, 0x0000, 0x0000)),
        (-0.0, (0x8000, 0x8000, 0x8000)),
        (math.inf, (0x7F80, 0x7F80, 0x7F80)),
        (-math.inf, (0xFF80, 0xFF80, 0xFF80)),
        (bmax, (0x7F7F, 0x7F7F, 0x7F7F)),
        (bmax + ulp_max / 2, (0x7F80, 0x7F80, 0x7F7F)),  # tie above the maximum
        (-(bmax + ulp_max / 4), (0xFF7F, 0xFF7F, 0xFF7F)),
        (1e300, (0x7F80, 0x7F80, 0x7F7F)),
        (-1e300, (0xFF80, 0xFF80, 0xFF7F)),
        (2.0**-133, (0x0001, 0x0001, 0x0001)),  # smallest bf16 subnormal
        (2.0**-134, (0x0000, 0x0001, 0x0000)),  # half of it: a tie at zero
        (3 * 2.0**-135, (0x0001, 0x0001, 0x0000)),
        (5e-324, (0x0000, 0x0000, 0x0000)),
    ]
    for x, want in cases:
        for mode, w in zip(MODES, want):
            assert int(oracle.round_bf16(np.array([x]), mode)[0]) == w, (x, mode)
    for mode in MODES:
        assert int(oracle.round_bf16(np.array([math.nan]), mode)[0]) == 0x7FC0


@settings(max_examples=300, deadline=None)
@given(st.floats(allow_nan=False, allow_infinity=False, width=64), st.sampled_from(MODES))
def test_round_hypothesis(x, mode):
    assert int(oracle.round_bf16(np.array([x]), mode)[0]) == round_exact(x, mode)


def test_round_is_sign_symmetric():
    rng = np.random.default_rng(3)
    xs = rng.standard_normal(5000) * np.exp2(rng.integers(-130, 128, 5000))
    for mode in MODES:
        a = oracle.round_bf16(xs, mode)
        b = oracle.round_bf16(-xs, mode)
        assert np.array_equal(a ^ np.uint16(0x8000), b)
