"""GPU parity of the key-range-splitting entry point attn_fwd_bf16_ws.

The shapes below leave most compute units idle with one workgroup per 256
query rows, so the library splits their key ranges and merges the partial
rows in a second kernel.  Every row is checked against the fp64 oracle under
the row-scaled 2-ULP gate, in every rounding mode, plus the NaN/Inf rules
through the merge (a key range whose logits are all -Inf, a row with no
finite logit) and determinism.
"""
import numpy as np
import pytest
import torch

import bf16_forward_attention_amd as attn
import oracle
from bf16_forward_attention_amd import synth
from tests.gate import gate
from tests.gpu_util import MODES, Dev, launch_ws, say, to_bits, to_device

pytestmark = pytest.mark.gpu

D = 128
BF16_ONE, BF16_NINF = 0x3F80, 0xFF80


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


SPLIT_SHAPES = [(1, 1, 300, 3000), (2, 3, 200, 5000), (1, 2, 1, 4097), (1, 1, 513, 2048), (3, 1, 64, 640)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_split_shapes_all_modes(shape, layout):
    B, H, Sq, Sk = shape
    assert attn.attn_fwd_bf16_workspace_size(B, H, Sq, Sk) > 0, "shape expected to split"
    inp = synth.small(B, H, Sq, Sk, layout, seed=Sq * 13 + Sk)
    ex, rd = oracle.attn_all(inp.q, inp.k, inp.v, layout)
    dev = Dev(inp)
    for m, mode in enumerate(MODES):
        got = dev.run_logical(mode, split=True)
        res = gate(got, rd[m], ex)
        say(f"  split {shape} {layout} {mode}: {res.summary()}")
        assert res.ok, res.summary()
    again = dev.run_logical("rtne", split=True)
    assert np.array_equal(again, dev.run_logical("rtne", split=True)), "split path not deterministic"


def test_no_split_when_the_grid_is_full():
    # 2048 work items on 256 compute units: attn_fwd_bf16_ws is attn_fwd_bf16
    assert attn.attn_fwd_bf16_workspace_size(4, 16, 8192, 8192) == 0
    inp = synth.small(1, 256, 256, 300, "bhsd", seed=5)
    assert attn.attn_fwd_bf16_workspace_size(1, 256, 256, 300) == 0
    dev = Dev(inp)
    assert np.array_equal(dev.run("rtna", split=True), dev.run("rtna", split=False))


def test_stressed_logits_through_the_merge():
    B, H, Sq, Sk = 1, 2, 200, 4000
    inp = synth.small(B, H, Sq, Sk, "bshd", seed=11, qk_sigma=2.0, v_dist="uniform")
    q = synth.to_logical(inp.q, "bshd").copy()
    q[:, :, :7] = (((q[:, :, :7].astype(np.uint32) << 16).view(np.float32) * 64).view(np.uint32) >> 16).astype(np.uint16)
    qq = synth.to_layout(q, "bshd")
    ex, rd = oracle.attn_all(qq, inp.k, inp.v, "bshd")
    dq, dk, dv = to_device(qq), to_device(inp.k), to_device(inp.v)
    o = torch.empty_like(dq)
    for m, mode in enumerate(MODES):
        assert launch_ws(dq, dk, dv, o, "bshd", mode) > 0
        got = np.ascontiguousarray(synth.to_logical(to_bits(o), "bshd"))
        res = gate(got, rd[m], ex)
        say(f"  stressed split {mode}: {res.summary()}")
        assert res.ok, res.summary()


def _run_specials(B, H, Sq, Sk, q, k, v, layout="bhsd"):
    qq, kk = synth.to_layout(q, layout), synth.to_layout(k, layout)
    assert attn.attn_fwd_bf16_workspace_size(B, H, Sq, Sk) > 0
    ex, rd = oracle.attn_all(qq, kk, v, layout)
    dq, dk, dv = to_device(qq), to_device(kk), to_device(v)
    o = torch.empty_like(dq)
    outs = []
    for m, mode in enumerate(MODES):
        launch_ws(dq, dk, dv, o, layout, mode)
        got = np.ascontiguousarray(synth.to_logical(to_bits(o), layout))
        res = gate(got, rd[m], ex)
        say(f"  specials {mode}: {res.summary()}")
        assert res.ok, res.summary()
        outs.append(got)
    return outs


def test_minus_inf_key_ranges():
    # Rows 0..99 have q[0] = 1 and keys 0..1999 have k[0] = -Inf: those keys
    # drop out, so whole key ranges of those rows hold no finite logit.  Rows
    # 100..149 keep a random q[0]: a negative one meets -Inf * q[0] = +Inf
    # (NaN row), a positive one drops the same keys.
    B, H, Sq, Sk = 1, 1, 150, 2500
    inp = synth.small(B, H, Sq, Sk, "bhsd", seed=3)
    q = synth.to_logical(inp.q, "bhsd").copy()
    k = synth.to_logical(inp.k, "bhsd").copy()
    q[0, 0, :100, 0] = BF16_ONE
    k[0, 0, :2000, 0] = BF16_NINF
    got = _run_specials(B, H, Sq, Sk, q, k, inp.v)[0]
    nan_rows = np.all((got[0, 0] & 0x7FFF) > 0x7F80, axis=-1)
    assert not nan_rows[:100].any()
    q0 = (q[0, 0, 100:, 0].astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(nan_rows[100:], q0 <= 0)  # +Inf logit or 0 * -Inf


def test_rows_without_a_finite_logit():
    # every key has k[0] = -Inf and every row q[0] = 1: no finite logit
    # anywhere, every range reports m = -FLT_MAX and l = 0, every row is NaN
    B, H, Sq, Sk = 1, 1, 40, 1000
    inp = synth.small(B, H, Sq, Sk, "bhsd", seed=4)
    q = synth.to_logical(inp.q, "bhsd").copy()
    k = synth.to_logical(inp.k, "bhsd").copy()
    q[0, 0, :, 0] = BF16_ONE
    k[0, 0, :, 0] = BF16_NINF
    for got in _run_specials(B, H, Sq, Sk, q, k, inp.v):
        assert np.all((got & 0x7FFF) > 0x7F80)


def test_workspace_errors_on_device():
    inp = synth.small(1, 1, 300, 3000, "bshd", seed=1)
    dq, dk, dv = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    o = torch.empty_like(dq)
    need = attn.attn_fwd_bf16_workspace_size(1, 1, 300, 3000)
    ws = torch.empty(need + 64, dtype=torch.uint8, device="cuda:0")
    s = torch.cuda.current_stream().cuda_stream
    args = (dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), o.data_ptr(), 1, 1, 300, 3000, 0, 0)
    assert attn.attn_fwd_bf16_ws(*args, 0, need, s) == 1  # ATTN_ERR_NULL
    assert attn.attn_fwd_bf16_ws(*args, ws.data_ptr(), need - 1, s) == 9  # ATTN_ERR_WORKSPACE
    assert attn.attn_fwd_bf16_ws(*args, ws.data_ptr() + 8, need, s) == 5  # ATTN_ERR_ALIGN
    assert attn.attn_fwd_bf16_ws(*args, dq.data_ptr(), need, s) == 6  # ATTN_ERR_ALIAS (workspace over q)
    assert attn.attn_fwd_bf16_ws(*args, ws.data_ptr(), need, s) == 0
    torch.cuda.synchronize()


# decode-like shapes: a few query rows against a long key cache. They leave most compute units
# idle, so the splitting entry points cut the keys into ranges; each shape is checked single pass
# and split, unmasked in every mode, and with the bottom-right causal mask (each new query sees
# the cache and the new keys up to its own position) through attn_fwd_bf16_gqa_ws.
DECODE_SHAPES = [(1, 8, 1, 131072), (2, 4, 16, 65537), (1, 16, 7, 40000)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_like_long_key_caches(shape):
    B, H, Sq, Sk = shape
    assert attn.attn_fwd_bf16_workspace_size(B, H, Sq, Sk) > 0, "shape expected to split"
    inp = synth.small(B, H, Sq, Sk, "bshd", seed=Sk + Sq)
    ex, rd = oracle.attn_all(inp.q, inp.k, inp.v, "bshd")
    dev = Dev(inp)
    for split in (False, True):
        for m, mode in enumerate(MODES):
            res = gate(dev.run_logical(mode, split=split), rd[m], ex)
            say(f"  decode {shape} split={split} {mode}: {res.summary()}")
            assert res.ok, res.summary()
    ex, rd = oracle.attn_all(inp.q, inp.k, inp.v, "bshd", mask="causal_br")
    for split in (False, True):
        res = gate(dev.run_logical("rtna", split=split, mask="causal_br"), rd[1], ex)
        say(f"  decode {shape} causal_br split={split} rtna: {res.summary()}")
        assert res.ok, res.summary()


@pytest.mark.timeout(300)
def test_one_key_against_many_query_rows():
    # every row's only weight is exp2(<= 0) rounded to 1, so every output row is V's one row,
    # bit for bit, in every mode; 70001 rows over two heads (274 work items, a ragged last q-tile)
    inp = synth.small(1, 2, 70001, 1, "bhsd", seed=77)
    dev = Dev(inp)
    v = synth.to_logical(inp.v, "bhsd")
    for mode in MODES:
        got = dev.run_logical(mode, split=True)
        for h in range(2):
            assert np.array_equal(got[0, h], np.broadcast_to(v[0, h, 0], got[0, h].shape)), (mode, h)
