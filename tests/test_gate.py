"""CPU checks of the parity gate itself."""
import numpy as np

import oracle
from bf16_forward_attention_amd import synth
from tests.gate import gate, merge, row_ulp


def _oracle_rows():
    inp = synth.small(1, 2, 8, 50, "bhsd", seed=4)
    ex, rd = oracle.attn_all(inp.q, inp.k, inp.v, "bhsd")
    return ex, rd


def test_identical_passes():
    ex, rd = _oracle_rows()
    for m in range(3):
        res = gate(rd[m], rd[m], ex)
        assert res.ok and res.violations == 0 and res.strict_hist[">2"] == 0


def test_row_scaled_tolerance_edges():
    ex, rd = _oracle_rows()
    ulp = row_ulp(ex)
    vals = (rd[0].astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    # move one element by 2 row-ulps (allowed) and by 3 row-ulps (not allowed)
    for shift, ok in ((2.0, True), (3.0, False)):
        moved = vals.copy()
        moved[0, 1, 3, 7] += shift * ulp[0, 1, 3, 0]
        bits = (moved.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        assert np.array_equal(bits[0, 1, 3, 7:8] != rd[0][0, 1, 3, 7:8], [True])
        assert gate(bits, rd[0], ex).ok == ok


def test_nan_and_inf_positions_must_match():
    ex, rd = _oracle_rows()
    g = rd[1].copy()
    g[0, 0, 2, 5] = 0x7FC0
    assert gate(g, rd[1], ex).nan_mismatch == 1
    g = rd[1].copy()
    g[0, 0, 2, 5] = 0x7F80
    assert gate(g, rd[1], ex).inf_mismatch == 1


def _fp32_kernel_model(q_bits, k_bits, v_bits, mode, p_rounding):
    """A numpy stand-in for an fp32-accumulating attention kernel on one head
    (logical [S, 128] bf16 bits): fp32 logits, base-2 softmax against the row
    maximum, the row sum from the unrounded weights, the weights rounded to bf16
    (``p_rounding``: "rne" or "trunc") for the second product, one division and
    one rounding of the fp32 output to bf16 in ``mode``."""
    f = lambda b: (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    q, k, v = f(q_bits), f(k_bits), f(v_bits)
    t = (q @ k.T) * np.float32(np.log2(np.e) / np.sqrt(128.0))
    p = np.exp2(t - t.max(axis=1, keepdims=True)).astype(np.float32)
    l = p.sum(axis=1, keepdims=True, dtype=np.float32)
    u = p.view(np.uint32)
    if p_rounding == "rne":
        u = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    pb = (u & np.uint32(0xFFFF0000)).view(np.float32)
    o = ((pb @ v) / l).astype(np.float32).view(np.uint32)
    if mode == "rtne":
        o = o + np.uint32(0x7FFF) + ((o >> np.uint32(16)) & np.uint32(1))
    elif mode == "rtna":
        o = o + np.uint32(0x8000)
    return (o >> np.uint32(16)).astype(np.uint16)


def test_rms_guard_separates_unbiased_from_truncated_weights():
    # the guard must pass a kernel that rounds the weights to nearest and fail one that truncates them
    # (weights biased low by about 2^-9 on average, not compensated in the row sum), in every mode
    inp = synth.small(1, 1, 256, 2048, "bhsd", seed=9)
    ex, rd = oracle.attn_all(inp.q, inp.k, inp.v, "bhsd")
    for m, mode in enumerate(("rtne", "rtna", "rtz")):
        good = _fp32_kernel_model(inp.q[0, 0], inp.k[0, 0], inp.v[0, 0], mode, "rne")
        bad = _fp32_kernel_model(inp.q[0, 0], inp.k[0, 0], inp.v[0, 0], mode, "trunc")
        rg, rb = gate(good, rd[m][0, 0], ex[0, 0]), gate(bad, rd[m][0, 0], ex[0, 0])
        assert rg.ok and rg.rms_guard_ok, (mode, rg.summary())
        assert rg.rms_excess < 2.0e-3, (mode, rg.summary())
        assert not rb.rms_guard_ok, (mode, rb.summary())


def test_merge_of_row_chunks_equals_one_gate():
    ex, rd = _oracle_rows()
    g = rd[0].copy()
    g[0, 1, 4, 9] ^= 1
    whole = gate(g, rd[0], ex)
    parts = merge([gate(g[:, h], rd[0][:, h], ex[:, h]) for h in range(2)])
    assert (parts.n, parts.violations, parts.strict_hist, parts.rms_floor_violations) == \
        (whole.n, whole.violations, whole.strict_hist, whole.rms_floor_violations)
    assert abs(parts.rms_rel - whole.rms_rel) < 1e-12 and abs(parts.rms_excess - whole.rms_excess) < 1e-12
