"""GPU parity of the per-row log-sum-exp (the lse output of attn_fwd_bf16_gqa
and attn_fwd_bf16_varlen) against the oracle, within the bound
tests.gate.lse_tolerance derives from the fp32 arithmetic, with identical
NaN / -Inf positions; asking for it must not change a bit of the output."""
import math

import numpy as np
import pytest
import torch

import bf16_forward_attention_amd as attn
import oracle
from bf16_forward_attention_amd import synth
from tests import cases
from tests.gate import lse_gate, lse_tolerance
from tests.gpu_util import launch_gqa, say, to_bits, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


def _bound_inputs(q_log, k_log, mask, Sq, Sk):
    """max_j sum_c |q_c k_jc| / sqrt(128) over each row's visible keys, and their count."""
    H, H_kv = q_log.shape[1], k_log.shape[1]
    qa = np.abs(cases.val(q_log))
    ka = np.repeat(np.abs(cases.val(k_log)), H // H_kv, axis=1)
    dots = np.matmul(qa, np.ascontiguousarray(np.swapaxes(ka, -1, -2))) / math.sqrt(128)
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    if mask == "none":
        vis = np.ones((Sq, Sk), bool)
    else:
        off = 0 if mask == "causal" else Sk - Sq
        vis = j <= i + off
    dots = np.where(vis, dots, 0.0)
    return dots.max(axis=-1, initial=0.0), np.broadcast_to(vis.sum(axis=-1), dots.shape[:-1])


@pytest.mark.parametrize("shape", [(1, 2, 2, 300, 300), (2, 4, 2, 257, 1000), (1, 2, 1, 700, 100)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("mask", ["none", "causal", "causal_br"])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_lse_all_rows(shape, mask, layout):
    B, H, H_kv, Sq, Sk = shape
    inp = synth.small(B, H, Sq, Sk, layout, seed=Sq + Sk + H_kv, qk_sigma=1.5, mask=mask, H_kv=H_kv)
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(Sq)]
    _, _, ref = oracle.attn_rows(inp.q, inp.k, inp.v, layout, rows, mask=mask, with_lse=True)
    ref = ref.reshape(B, H, Sq)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    lse = torch.full((B, H, Sq), 7.0, dtype=torch.float32, device="cuda:0")
    launch_gqa(q, k, v, o1, layout, "rtne", mask, lse=lse)
    launch_gqa(q, k, v, o2, layout, "rtne", mask)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(o1), to_bits(o2)), "asking for lse changed the output"
    dmax, nvis = _bound_inputs(synth.to_logical(inp.q, layout), synth.to_logical(inp.k, layout), mask, Sq, Sk)
    ok, worst, n = lse_gate(lse.cpu().numpy(), ref, lse_tolerance(dmax, nvis, ref))
    say(f"  lse {shape} {mask} {layout}: worst err/tol {worst:.3f} over {n} finite rows")
    assert ok, f"worst err/tol {worst:.3f}"


def test_lse_special_values():
    B, H, Sq, Sk = 1, 4, 130, 90
    inp = synth.small(B, H, Sq, Sk, "bhsd", seed=3)
    k = inp.k.copy()
    q = inp.q.copy()
    k[0, 0, 3, 5] = 0x7FC0                    # NaN logit: head 0 all NaN
    k[0, 1, 2, 7] = 0x7F80                    # +Inf: NaN rows where q[., 7] > 0
    q[0, 2, :, 0] = cases.bf(1.0)
    k[0, 2, :, 0] = 0xFF80                    # head 2: every logit -Inf
    rows = [(0, h, i) for h in range(H) for i in range(Sq)]
    _, _, ref = oracle.attn_rows(q, k, inp.v, "bhsd", rows, with_lse=True)
    ref = ref.reshape(B, H, Sq)
    dq, dk, dv = to_device(q), to_device(k), to_device(inp.v)
    o = torch.empty_like(dq)
    lse = torch.zeros((B, H, Sq), dtype=torch.float32, device="cuda:0")
    launch_gqa(dq, dk, dv, o, "bhsd", "rtne", "none", lse=lse)
    torch.cuda.synchronize()
    got = lse.cpu().numpy()
    assert np.all(np.isnan(got[0, 0])) and np.all(got[0, 2] == -np.inf)
    dmax, nvis = _bound_inputs(q, k, "none", Sq, Sk)
    ok, worst, n = lse_gate(got, ref, lse_tolerance(np.nan_to_num(dmax, posinf=0.0), nvis, ref))
    assert ok, f"worst err/tol {worst:.3f}"


def test_lse_varlen():
    wl = synth.VarlenWorkload("lse_varlen", (300, 0, 40, 513), (280, 30, 0, 700), 4, 2, ("rtne",),
                              mask="causal_br", seed=9)
    inp = synth.generate_varlen(wl)
    tq = inp.q.shape[0]
    rows = [(t, h) for t in range(tq) for h in range(wl.H)]
    _, _, ref = oracle.attn_rows_varlen(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, rows, wl.mask, with_lse=True)
    ref = ref.reshape(tq, wl.H).T  # [H, total_q]
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    cq, ck = torch.from_numpy(inp.cu_q).to("cuda:0"), torch.from_numpy(inp.cu_k).to("cuda:0")
    o = torch.empty_like(q)
    lse = torch.zeros((wl.H, tq), dtype=torch.float32, device="cuda:0")
    st = attn.attn_fwd_bf16_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   cq.data_ptr(), ck.data_ptr(), wl.B, wl.H, wl.H_kv, tq, inp.k.shape[0],
                                   max(wl.lengths_q), 0, attn.MASKS[wl.mask], torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    got = lse.cpu().numpy()
    tol = np.full(ref.shape, 0.0)
    for b in range(wl.B):
        q0, q1, k0, k1 = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        if q1 == q0:
            continue
        ql = inp.q[q0:q1].transpose(1, 0, 2)[None]
        kl = inp.k[k0:k1].transpose(1, 0, 2)[None]
        if k1 == k0:
            continue
        dmax, nvis = _bound_inputs(ql, kl, wl.mask, q1 - q0, k1 - k0)
        tol[:, q0:q1] = lse_tolerance(dmax[0], nvis[0], ref[:, q0:q1])
    ok, worst, n = lse_gate(got, ref, tol)
    say(f"  lse varlen: worst err/tol {worst:.3f} over {n} finite rows")
    assert ok, f"worst err/tol {worst:.3f}"
