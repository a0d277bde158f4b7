"""CPU checks of the parity gate itself."""
import numpy as np

import oracle
from bf16_forward_attention_amd import synth
from tests.gate import gate, row_ulp


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
