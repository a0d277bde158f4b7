"""GPU parity of the causal masks (attn_fwd_bf16_masked) against the oracle.

The reading of the causal mask (the pages name it only as missing from the
kernel they describe): query row i attends to keys j <= i + off, off = 0
("causal") or Sk - Sq ("causal_br"); rows with no visible key are NaN.  Every
row is compared under the row-scaled 2-ULP gate with identical NaN/Inf
positions, the diagonal-dominant case bit for bit, and repeated launches must
give identical bits.
"""
import numpy as np
import pytest
import torch

import oracle
from bf16_forward_attention_amd import synth
from tests import cases
from tests.gate import gate
from tests.gpu_util import MODES, Dev, launch_masked, run_logical, say, to_bits

pytestmark = pytest.mark.gpu

MASKS = ("causal", "causal_br")
SHAPES = [
    (1, 1, 1, 1), (1, 1, 1, 77), (1, 1, 77, 1), (1, 2, 256, 256), (2, 1, 300, 300), (1, 2, 513, 513),
    (1, 2, 100, 700), (1, 2, 700, 100), (1, 3, 257, 1200), (2, 2, 600, 333), (1, 1, 1000, 1000),
]


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


def _check_all_rows(inp, modes=MODES):
    ex, rd = oracle.attn_all(inp.q, inp.k, inp.v, inp.wl.layout, mask=inp.wl.mask)
    dev = Dev(inp)
    outs = {}
    for mode in modes:
        got = dev.run_logical(mode)
        res = gate(got, rd[MODES.index(mode)], ex)
        say(f"  {inp.wl.name} {mode}: {res.summary()}")
        assert res.ok, f"{inp.wl.name} {mode}: {res.summary()}"
        outs[mode] = got
    assert np.array_equal(dev.run_logical(modes[0]), outs[modes[0]]), "repeated launch changed the output"
    return outs


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("mask", MASKS)
def test_causal_shapes(shape, layout, mask):
    B, H, Sq, Sk = shape
    _check_all_rows(synth.small(B, H, Sq, Sk, layout, seed=Sq * 5 + Sk, mask=mask))


@pytest.mark.parametrize("mask", MASKS)
def test_rows_without_keys_are_nan(mask):
    # bottom right with Sq > Sk: rows i < Sq - Sk see no key
    B, H, Sq, Sk = 1, 2, 700, 100
    inp = synth.small(B, H, Sq, Sk, "bhsd", seed=3, mask=mask)
    got = Dev(inp).run_logical("rtne")
    nan_rows = np.all((got & 0x7FFF) > 0x7F80, axis=-1)
    any_nan = np.any((got & 0x7FFF) > 0x7F80, axis=-1)
    assert np.array_equal(nan_rows, any_nan)
    expect = np.arange(Sq) < (Sq - Sk if mask == "causal_br" else 0)
    assert np.array_equal(nan_rows, np.broadcast_to(expect, nan_rows.shape))


@pytest.mark.parametrize("shape", [(100, 100), (127, 300), (60, 1000), (127, 65)], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mask", MASKS)
def test_diagonal_key_bit_exact(shape, mask):
    # row i's key i + off dominates every other visible key: O_i = V_{i+off} exactly
    Sq, Sk = shape
    off = 0 if mask == "causal" else Sk - Sq
    q, k, v = cases.diagonal_dominant(1, 2, Sq, Sk, off, seed=Sq + Sk)
    for layout in ("bshd", "bhsd"):
        for mode in MODES:
            got = run_logical(q, k, v, layout, mode, mask)
            for i in range(Sq):
                if 0 <= i + off < Sk:
                    assert np.array_equal(got[:, :, i], v[:, :, i + off]), (layout, mode, i)


def test_none_mask_matches_unmasked_entry_point():
    inp = synth.small(1, 2, 300, 500, "bshd", seed=9)
    dev = Dev(inp)
    for mode in ("rtna", "rtz"):
        want = dev.run(mode)
        dev.o.zero_()
        launch_masked(dev.q, dev.k, dev.v, dev.o, "bshd", mode, "none")
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(dev.o), want), mode


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("shape", [(2, 37, 37, 1700, 1700, "bshd"), (1, 74, 37, 1700, 1900, "bhsd"),
                                   (1, 64, 16, 2048, 1500, "bshd")],
                         ids=["odd_qtiles", "odd_qtiles_gqa_longer_keys", "even_qtiles_gqa_shorter_keys"])
def test_paired_workgroups(shape, mask):
    # enough causal work items for two rounds of compute units: each workgroup runs q-tiles n-1-j and j
    # of a head one after the other (7 q-tiles per head leave the middle one alone); every row against
    # the oracle, and the lse of the rows of both items of a workgroup
    from tests.gate import lse_gate, lse_tolerance
    from tests.gpu_util import launch_gqa, to_device
    B, H, H_kv, Sq, Sk, layout = shape
    n_qtiles = -(-Sq // 256)
    assert B * H * n_qtiles >= 2 * torch.cuda.get_device_properties(0).multi_processor_count
    inp = synth.small(B, H, Sq, Sk, layout, seed=Sq + H, mask=mask, H_kv=H_kv)
    ex, rd, ls = oracle.attn_rows(inp.q, inp.k, inp.v, layout,
                                  [(b, h, i) for b in range(B) for h in range(H) for i in range(Sq)],
                                  mask=mask, with_lse=True)
    ex = ex.reshape(B, H, Sq, 128)
    rd = rd.reshape(B, H, Sq, 3, 128)
    ls = ls.reshape(B, H, Sq)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda:0")
    for m, mode in enumerate(MODES):
        launch_gqa(q, k, v, o, layout, mode, mask, lse=lse)
        torch.cuda.synchronize()
        got = np.ascontiguousarray(synth.to_logical(to_bits(o), layout))
        res = gate(got, rd[:, :, :, m], ex)
        say(f"  {shape} {mask} {mode}: {res.summary()}")
        assert res.ok, (mode, res.summary())
    # lse against the oracle's, within the bound derived from the fp32 arithmetic
    from tests.test_gpu_lse import _bound_inputs
    ql, kl = synth.to_logical(inp.q, layout), synth.to_logical(inp.k, layout)
    got = lse.cpu().numpy()
    for b in range(B):
        dmax, nvis = _bound_inputs(ql[b:b + 1], kl[b:b + 1], mask, Sq, Sk)
        ok, worst, n = lse_gate(got[b:b + 1], ls[b:b + 1], lse_tolerance(dmax, nvis, ls[b:b + 1]))
        say(f"  lse batch {b}: worst {worst:.3f} of the bound over {n} rows")
        assert ok, worst
