"""GPU parity of attn_fwd_bf16_gqa_ws: the split of key ranges under the
causal masks, with grouped K/V heads and with the log-sum-exp output.

Under a causal mask a work item (256 query rows of one head) visits the key
tiles up to its last row's limit.  When the items are nearly equal (a short
Sq against a long Sk, diagonal at the bottom right) and do not fill the last
round of compute units, each item of that round cuts its visible tiles into
consecutive ranges and a second kernel merges the partial rows; when they
are unequal and all fit in one round, every item is cut.  Every row is
checked against the fp64 oracle under the row-scaled 2-ULP gate in every
rounding mode, the lse within its fp32 bound, and repeated calls for
identical bits; items that run whole must give exactly the single-pass bits.
"""
import math

import numpy as np
import pytest
import torch

import bf16_forward_attention_amd as attn
import oracle
from bf16_forward_attention_amd import synth
from tests import cases
from tests.gate import gate, lse_gate, lse_tolerance
from tests.gpu_util import MODES, launch_gqa, launch_gqa_ws, say, to_bits, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


def _n_cu():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _lse_bound(q_log, k_log, mask, Sq, Sk):
    """max_j sum_c |q_c k_jc| / sqrt(128) over each row's visible keys, and their count."""
    H, H_kv = q_log.shape[1], k_log.shape[1]
    qa = np.abs(cases.val(q_log))
    ka = np.repeat(np.abs(cases.val(k_log)), H // H_kv, axis=1)
    dots = np.einsum("bhid,bhjd->bhij", qa, ka) / math.sqrt(128)
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    vis = np.ones((Sq, Sk), bool) if mask == "none" else j <= i + (0 if mask == "causal" else Sk - Sq)
    dots = np.where(vis, dots, 0.0)
    return dots.max(axis=-1, initial=0.0), np.broadcast_to(vis.sum(axis=-1), dots.shape[:-1])


# (B, H, H_kv, Sq, Sk, mask)
SHAPES = [
    (1, 4, 4, 300, 2000, "causal_br"),   # 8 items of 31-32 tiles: 8 ranges each
    (1, 24, 24, 512, 1280, "causal_br"),  # 48 items x 5 ranges; the q-tiles that see 16 tiles leave one range empty
    (1, 8, 2, 300, 2000, "causal_br"),   # grouped K/V heads
    (2, 4, 1, 300, 2000, "none"),        # multi-query heads, no mask
    (1, 3, 3, 1000, 7000, "causal_br"),  # ragged last q-tile (232 rows)
    # one round of unequal items (top-left diagonal, few heads): every item cut into ranges
    (1, 2, 2, 1000, 1000, "causal"),     # 8 items of 4 .. 16 tiles, 4 ranges each (some empty)
    (1, 3, 1, 777, 2500, "causal"),      # 12 items of 4 .. 13 tiles, 3 ranges each
    (2, 2, 1, 1500, 1500, "causal_br"),  # Sq = Sk: the bottom-right diagonal is the top-left one
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:5])) + "_" + s[5])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_split_masked_all_modes(shape, layout):
    B, H, H_kv, Sq, Sk, mask = shape
    whole, items, splits, _ = attn.attn_fwd_bf16_split_plan_masked(B * H, Sq, Sk, attn.MASKS[mask], _n_cu())
    assert items > 0, "shape expected to split"
    inp = synth.small(B, H, Sq, Sk, layout, seed=Sq * 7 + Sk + H_kv, qk_sigma=1.5, mask=mask, H_kv=H_kv)
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(Sq)]
    ex, rd, ref_lse = oracle.attn_rows(inp.q, inp.k, inp.v, layout, rows, mask=mask, with_lse=True)
    ex = ex.reshape(B, H, Sq, 128)
    rd = np.moveaxis(rd.reshape(B, H, Sq, 3, 128), 3, 0)
    ref_lse = ref_lse.reshape(B, H, Sq)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    o = torch.empty_like(q)
    lse = torch.full((B, H, Sq), 7.0, dtype=torch.float32, device="cuda:0")
    first = None
    for m, mode in enumerate(MODES):
        assert launch_gqa_ws(q, k, v, o, layout, mode, mask, lse=lse) > 0
        got = np.ascontiguousarray(synth.to_logical(to_bits(o), layout))
        res = gate(got, rd[m], ex)
        say(f"  split {shape} {layout} {mode} ({whole} whole, {items} x {splits}): {res.summary()}")
        assert res.ok, res.summary()
        if m == 0:
            first = got
            dmax, nvis = _lse_bound(synth.to_logical(inp.q, layout), synth.to_logical(inp.k, layout), mask, Sq, Sk)
            ok, worst, n = lse_gate(lse.cpu().numpy(), ref_lse, lse_tolerance(dmax, nvis, ref_lse))
            say(f"  lse worst err/tol {worst:.3f} over {n} rows")
            assert ok, f"lse worst err/tol {worst:.3f}"
    launch_gqa_ws(q, k, v, o, layout, MODES[0], mask)
    again = np.ascontiguousarray(synth.to_logical(to_bits(o), layout))
    assert np.array_equal(first, again), "split path not deterministic (or lse changed the output)"


def test_whole_items_keep_the_single_pass_bits():
    # 132 heads of 2 q-tiles = 264 items: 256 run whole, the last 8 (heads 128..131)
    # as 8 ranges each
    B, H, Sq, Sk, mask = 1, 132, 300, 2000, "causal_br"
    whole, items, splits, _ = attn.attn_fwd_bf16_split_plan_masked(B * H, Sq, Sk, attn.MASKS[mask], _n_cu())
    if _n_cu() != 256:
        pytest.skip("item counts below assume 256 compute units")
    assert (whole, items) == (256, 8) and splits >= 2
    inp = synth.small(B, H, Sq, Sk, "bshd", seed=41, mask=mask)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    o_ws, o_one = torch.empty_like(q), torch.empty_like(q)
    launch_gqa_ws(q, k, v, o_ws, "bshd", "rtna", mask)
    launch_gqa(q, k, v, o_one, "bshd", "rtna", mask)
    torch.cuda.synchronize()
    got = synth.to_logical(to_bits(o_ws), "bshd")
    one = synth.to_logical(to_bits(o_one), "bshd")
    assert np.array_equal(got[:, :128], one[:, :128]), "whole items differ from the single pass"
    rows = [(0, h, i) for h in range(128, 132) for i in range(Sq)]
    ex, rd = oracle.attn_rows(inp.q, inp.k, inp.v, "bshd", rows, mask=mask)
    res = gate(got[0, 128:].reshape(-1, 128), rd[:, 1], ex)
    say(f"  split items: {res.summary()}")
    assert res.ok, res.summary()


@pytest.mark.parametrize("shape", [(1, 96, 96, 700, 700, "causal"), (2, 4, 2, 300, 2000, "causal"),
                                   (1, 4, 4, 2000, 300, "causal_br")], ids=lambda s: "x".join(map(str, s[:5])) + s[5])
def test_unequal_items_run_single_pass(shape):
    # the q-tiles of a head see very different key counts: over more than one
    # round of items (288 here) the longest-first order keeps the CUs busy, and
    # items of at most 7 tiles are too short to cut, so nothing is split and the
    # call is attn_fwd_bf16_gqa exactly
    B, H, H_kv, Sq, Sk, mask = shape
    assert attn.attn_fwd_bf16_gqa_workspace_size(B, H, Sq, Sk, attn.MASKS[mask]) == 0
    inp = synth.small(B, H, Sq, Sk, "bhsd", seed=3, mask=mask, H_kv=H_kv)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    o_ws, o_one = torch.empty_like(q), torch.empty_like(q)
    assert launch_gqa_ws(q, k, v, o_ws, "bhsd", "rtz", mask) == 0
    launch_gqa(q, k, v, o_one, "bhsd", "rtz", mask)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(o_ws), to_bits(o_one))


def test_binding_splits_masked_calls():
    B, H, Sq, Sk = 1, 4, 300, 2000
    inp = synth.small(B, H, Sq, Sk, "bshd", seed=8, mask="causal_br")
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    out, lse = attn.attn_fwd(q, k, v, layout="bshd", round_mode="rtne", mask="causal_br", with_lse=True)
    o_ws = torch.empty_like(q)
    lse_ws = torch.empty_like(lse)
    launch_gqa_ws(q, k, v, o_ws, "bshd", "rtne", "causal_br", lse=lse_ws)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), to_bits(o_ws))
    assert np.array_equal(lse.cpu().numpy().view(np.uint32), lse_ws.cpu().numpy().view(np.uint32))


def test_workspace_errors_on_device():
    B, H, Sq, Sk, mask = 1, 4, 300, 2000, attn.MASKS["causal_br"]
    need = attn.attn_fwd_bf16_gqa_workspace_size(B, H, Sq, Sk, mask)
    assert need > 0
    dq = torch.zeros((B, Sq, H, 128), dtype=torch.bfloat16, device="cuda:0")
    dk = torch.zeros((B, Sk, H, 128), dtype=torch.bfloat16, device="cuda:0")
    o = torch.empty_like(dq)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    s = torch.cuda.current_stream().cuda_stream
    args = (dq.data_ptr(), dk.data_ptr(), dk.data_ptr(), o.data_ptr(), 0, B, H, H, Sq, Sk, 0, 0, mask)
    assert attn.attn_fwd_bf16_gqa_ws(*args, 0, need, s) == 1          # ATTN_ERR_NULL
    assert attn.attn_fwd_bf16_gqa_ws(*args, ws.data_ptr(), need - 1, s) == 9  # ATTN_ERR_WORKSPACE
    assert attn.attn_fwd_bf16_gqa_ws(*args, ws.data_ptr() + 4, need, s) == 5  # ATTN_ERR_ALIGN
    assert attn.attn_fwd_bf16_gqa_ws(*args, o.data_ptr(), need, s) == 6       # ATTN_ERR_ALIAS
    assert attn.attn_fwd_bf16_gqa_ws(*args, ws.data_ptr(), need, s) == 0
    torch.cuda.synchronize()


def test_split_writes_stay_inside_o_and_lse():
    # o and lse carved out of larger buffers filled with sentinels: the split kernel, the merge and
    # the lse stores touch nothing outside them (the ragged last q-tile's rows >= Sq included)
    B, H, Sq, Sk, mask = 1, 4, 300, 2000, "causal_br"
    inp = synth.small(B, H, Sq, Sk, "bshd", seed=61, mask=mask)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    pad = 4096  # elements on each side
    n_o, n_l = q.numel(), B * H * Sq
    o_buf = torch.full((n_o + 2 * pad,), 0x7E7E, dtype=torch.int16, device="cuda:0")
    l_buf = torch.full((n_l + 2 * pad,), -12345.0, dtype=torch.float32, device="cuda:0")
    o = o_buf[pad:pad + n_o].view(torch.bfloat16).view(q.shape)
    lse = l_buf[pad:pad + n_l].view(B, H, Sq)
    assert launch_gqa_ws(q, k, v, o, "bshd", "rtne", mask, lse=lse) > 0
    ob, lb = o_buf.cpu().numpy(), l_buf.cpu().numpy()
    assert np.all(ob[:pad] == 0x7E7E) and np.all(ob[pad + n_o:] == 0x7E7E)
    assert np.all(lb[:pad] == -12345.0) and np.all(lb[pad + n_l:] == -12345.0)
    assert np.all(np.isfinite(lb[pad:pad + n_l]))
