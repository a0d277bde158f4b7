"""GPU parity at sizes where the oracle computes every row.

Each case compares the HIP library (called through its C ABI) with the fp64
oracle element by element under the row-scaled 2-ULP gate (tests/gate.py),
or bit for bit where the exact result is representable.
"""
import numpy as np
import pytest
import torch

import oracle
from bf16_forward_attention_amd import synth
from tests import cases
from tests.gate import gate
from tests.gpu_util import MODES, Dev, launch, run_logical, run_raw, say, to_bits, to_device

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


def _check_all_rows(inp, modes=MODES):
    ex, rd = oracle.attn_all(inp.q, inp.k, inp.v, inp.wl.layout)
    dev = Dev(inp)
    for mode in modes:
        m = MODES.index(mode)
        got = dev.run_logical(mode)
        res = gate(got, rd[m], ex)
        say(f"  {inp.wl.name} {mode}: {res.summary()}")
        assert res.ok, f"{inp.wl.name} {mode}: {res.summary()}"


def test_tiny_config_all_modes():
    # B=1, H=2, Sq=Sk=256, BHSD, N(0,1), seed 0, every rounding mode
    _check_all_rows(synth.generate(synth.WORKLOADS["tiny"]))


SHAPES = [
    (1, 1, 1, 1), (1, 1, 1, 65), (1, 2, 17, 1), (2, 3, 63, 64), (1, 2, 65, 127), (1, 1, 128, 129),
    (2, 2, 129, 200), (1, 3, 300, 63), (1, 1, 257, 1000), (1, 1, 4097, 96), (3, 1, 31, 2049),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_ragged_shapes(shape, layout):
    B, H, Sq, Sk = shape
    _check_all_rows(synth.small(B, H, Sq, Sk, layout, seed=Sq * 7 + Sk))


@pytest.mark.parametrize("Sk", [64 * 3 + 1, 64 * 3 + 3, 64 * 5 + 56, 64 * 2 + 63, 64, 1])
def test_dominant_key_bit_exact_including_tail_tile(Sk):
    q, k, v, jstar = cases.dominant(1, 2, 130, Sk, seed=Sk)
    for layout in ("bshd", "bhsd"):
        for mode in MODES:
            got = run_logical(q, k, v, layout, mode)
            for h in range(2):
                want = v[0, h, jstar[0, h]]
                assert np.array_equal(got[0, h], want), (layout, mode, h)


@pytest.mark.parametrize("row", [i for i, r in enumerate(cases.load_ties()) if r[2] == "both"])
def test_midpoint_ties_bit_exact(row):
    vals, want, _ = cases.load_ties()[row]
    q, k, v = cases.tie_inputs(vals)
    for m, mode in enumerate(MODES):
        got = run_logical(q, k, v, "bhsd", mode)
        assert np.all(got == want[m]), (vals, mode, got[0, 0, 0, :4])


def test_layouts_give_identical_bits():
    inp_s = synth.small(2, 3, 200, 333, "bshd", seed=1)
    inp_h = synth.small(2, 3, 200, 333, "bhsd", seed=1)
    for mode in MODES:
        a = Dev(inp_s).run_logical(mode)
        b = Dev(inp_h).run_logical(mode)
        assert np.array_equal(a, b), mode


def test_deterministic_across_runs():
    inp = synth.small(2, 4, 515, 2100, "bshd", seed=2)
    dev = Dev(inp)
    for mode in MODES:
        first = dev.run(mode)
        for _ in range(2):
            assert np.array_equal(dev.run(mode), first), mode


def test_negating_v_negates_o():
    inp = synth.small(1, 2, 150, 300, "bhsd", seed=3)
    for mode in MODES:
        a = run_raw(inp.q, inp.k, inp.v, "bhsd", mode)
        b = run_raw(inp.q, inp.k, inp.v ^ np.uint16(0x8000), "bhsd", mode)
        nan = ((a & 0x7FFF) > 0x7F80)
        assert np.array_equal((a ^ np.uint16(0x8000))[~nan], b[~nan]), mode


def test_single_key_returns_v0():
    q = cases.randn_bits((2, 3, 70, D), 8, sigma=3.0)
    k = cases.randn_bits((2, 3, 1, D), 9, sigma=3.0)
    v = cases.randn_bits((2, 3, 1, D), 10)
    for mode in MODES:
        got = run_logical(q, k, v, "bshd", mode)
        assert np.array_equal(got, np.broadcast_to(v, got.shape)), mode


def test_uniform_logits_mean_of_v():
    q = np.zeros((1, 2, 40, D), np.uint16)
    k = cases.randn_bits((1, 2, 777, D), 11)
    v = cases.randn_bits((1, 2, 777, D), 12)
    ex, rd = oracle.attn_all(q, k, v, "bhsd")
    for m, mode in enumerate(MODES):
        res = gate(run_logical(q, k, v, "bhsd", mode), rd[m], ex)
        assert res.ok, res.summary()


def _nan_inf_inputs():
    q = cases.randn_bits((1, 4, 70, D), 20)
    k = cases.randn_bits((1, 4, 150, D), 21)
    v = cases.randn_bits((1, 4, 150, D), 22)
    k[0, 0, 7, 33] = 0x7FC0      # NaN in K: head 0 all NaN
    k[0, 1, 70, 57] = 0x7F80     # +Inf in K: rows with q[57] > 0 are NaN
    k[0, 2, 149, 3] = 0xFF80     # -Inf in K, in the last (partial) tile
    q[0, 2, 5, 3] = 0            # 0 * Inf = NaN for that row
    q[0, 3, 9, 100] = 0xFFC1     # NaN in Q: one row
    return q, k, v


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_nan_inf_positions_match_oracle(layout):
    q, k, v = _nan_inf_inputs()
    ex, rd = oracle.attn_all(synth.to_layout(q, layout), synth.to_layout(k, layout), synth.to_layout(v, layout),
                             layout)
    assert np.isnan(ex).any() and np.isfinite(ex).any()
    for m, mode in enumerate(MODES):
        got = run_logical(q, k, v, layout, mode)
        res = gate(got, rd[m], ex)
        assert res.ok, (mode, res.summary())


def test_all_logits_minus_inf_give_nan_row():
    q = cases.randn_bits((1, 1, 3, D), 30)
    k = cases.randn_bits((1, 1, 130, D), 31)
    v = cases.randn_bits((1, 1, 130, D), 32)
    q[0, 0, :, 0] = cases.bf(1.0)
    k[0, 0, :, 0] = 0xFF80
    for mode in MODES:
        got = run_logical(q, k, v, "bhsd", mode)
        assert np.all((got & 0x7FFF) > 0x7F80), mode


def test_output_guard_bands_untouched():
    inp = synth.small(1, 2, 77, 90, "bshd", seed=5)
    dq, dk, dv = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    n = dq.numel()
    pad = 4096
    buf = torch.full((n + 2 * pad,), -12345, dtype=torch.int16, device="cuda:0")
    o = buf[pad:pad + n].view(torch.bfloat16).view(dq.shape)
    launch(dq, dk, dv, o, "bshd", "rtne")
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:pad] == -12345) and np.all(b[pad + n:] == -12345)
    ex, rd = oracle.attn_all(inp.q, inp.k, inp.v, "bshd")
    got = np.ascontiguousarray(synth.to_logical(to_bits(o), "bshd"))
    assert gate(got, rd[0], ex).ok


def test_runs_on_a_side_stream():
    inp = synth.small(1, 2, 300, 500, "bhsd", seed=6)
    ex, rd = oracle.attn_all(inp.q, inp.k, inp.v, "bhsd")
    dq, dk, dv = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    o = torch.empty_like(dq)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        launch(dq, dk, dv, o, "bhsd", "rtna", stream=s)
    s.synchronize()
    assert gate(to_bits(o), rd[1], ex).ok


def test_python_wrapper_matches_c_abi():
    import bf16_forward_attention_amd as attn
    inp = synth.small(2, 2, 100, 130, "bshd", seed=7)
    dev = Dev(inp)
    ref = dev.run("rtz")
    out = attn.attn_fwd(dev.q, dev.k, dev.v, layout="bshd", round_mode="rtz")
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(out), ref)
    with pytest.raises(ValueError):
        attn.attn_fwd(dev.q.float(), dev.k, dev.v)


def test_python_wrappers_on_a_caller_stream():
    # the torch-level calls enqueue on a stream the caller passes (not torch's current one) and
    # give the bits of the C ABI, with and without the log-sum-exp, fixed-length and packed
    import bf16_forward_attention_amd as attn
    inp = synth.small(2, 4, 300, 300, "bshd", seed=9)
    dev = Dev(inp)
    ref = dev.run("rtne")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    out = attn.attn_fwd(dev.q, dev.k, dev.v, layout="bshd", round_mode="rtne", stream=s, split=False)
    out2, lse = attn.attn_fwd(dev.q, dev.k, dev.v, layout="bshd", round_mode="rtne", stream=s, split=False,
                              with_lse=True)
    s.synchronize()
    assert np.array_equal(to_bits(out), ref)
    assert np.array_equal(to_bits(out2), ref)
    assert lse.shape == (2, 4, 300) and bool(torch.isfinite(lse).all())
    # the same rows packed as two sequences of 300
    qp, kp, vp = (t.reshape(600, 4, 128) for t in (dev.q, dev.k, dev.v))
    cu = torch.tensor([0, 300, 600], dtype=torch.int32, device=qp.device)
    outp = attn.attn_fwd_varlen(qp, kp, vp, cu, cu, 300, round_mode="rtne", stream=s)
    s.synchronize()
    assert np.array_equal(to_bits(outp).reshape(2, 300, 4, 128), ref)


def test_an_earlier_failed_hip_call_is_not_reported_as_a_launch_failure():
    # A HIP call of the caller that failed earlier (here hipSetDevice with a device index that does
    # not exist, rejected by the runtime on the host) can leave its error pending in the thread. The
    # library reports each launch's own status, so the next call succeeds all the same.
    import ctypes
    import bf16_forward_attention_amd as attn

    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    inp = synth.small(1, 2, 100, 130, "bshd", seed=8)
    ex, rd = oracle.attn_all(inp.q, inp.k, inp.v, "bshd")
    dev = Dev(inp)
    torch.cuda.synchronize()
    hip.hipGetLastError()  # start from a clean slate
    assert hip.hipSetDevice(1 << 20) != 0
    pending = hip.hipPeekAtLastError()
    say(f"  pending error after the failed call: {pending}")
    s = torch.cuda.current_stream()
    st = attn.attn_fwd_bf16(dev.q.data_ptr(), dev.k.data_ptr(), dev.v.data_ptr(), dev.o.data_ptr(), 1, 2, 100, 130,
                            attn.LAYOUTS["bshd"], attn.ROUND_MODES["rtne"], s.cuda_stream)
    hip.hipGetLastError()  # leave the thread clean for the tests that follow
    torch.cuda.synchronize()
    assert st == 0, attn.attn_fwd_bf16_strerror(st)
    got = np.ascontiguousarray(synth.to_logical(to_bits(dev.o), "bshd"))
    assert gate(got, rd[0], ex).ok
