"""GPU parity on a seeded random sweep of small problems.

Each case draws a layout, rounding mode, mask, batch, head counts (with
grouped K/V heads) and ragged query and key lengths, and runs the problem
through the single-pass entry point, the key-range-splitting one and, for a
random cut of the keys, through key shards and their merge; every output is
checked against the fp64 oracle under the row-scaled 2-ULP gate, the lse of
the split call within its fp32 bound.  The draws come from a fixed seed, so
the sweep is the same on every run.
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

N_CASES = 120


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    layout = ["bshd", "bhsd"][rng.integers(2)]
    mode = MODES[rng.integers(3)]
    mask = ["none", "causal", "causal_br"][rng.integers(3)]
    H_kv = int(rng.choice([1, 2, 3]))
    H = H_kv * int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 3))
    Sq = int(rng.choice([1, 2, 63, 64, 65, 200, 255, 256, 257, 511, 700]))
    Sk = int(rng.choice([1, 3, 63, 64, 65, 127, 300, 513, 1000, 1500]))
    return layout, mode, mask, B, H, H_kv, Sq, Sk


def _lse_bound(q_log, k_log, mask, Sq, Sk):
    H, H_kv = q_log.shape[1], k_log.shape[1]
    qa = np.abs(cases.val(q_log))
    ka = np.repeat(np.abs(cases.val(k_log)), H // H_kv, axis=1)
    dots = np.einsum("bhid,bhjd->bhij", qa, ka) / math.sqrt(128)
    i, j = np.arange(Sq)[:, None], np.arange(Sk)[None, :]
    vis = np.ones((Sq, Sk), bool) if mask == "none" else j <= i + (0 if mask == "causal" else Sk - Sq)
    dots = np.where(vis, dots, 0.0)
    return dots.max(axis=-1, initial=0.0), np.broadcast_to(vis.sum(axis=-1), dots.shape[:-1])


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    layout, mode, mask, B, H, H_kv, Sq, Sk = _draw(i)
    say(f"  case {i}: {layout} {mode} {mask} B={B} H={H} H_kv={H_kv} Sq={Sq} Sk={Sk}")
    inp = synth.small(B, H, Sq, Sk, layout, seed=7000 + i, qk_sigma=1.3, mask=mask, H_kv=H_kv)
    rows = [(b, h, r) for b in range(B) for h in range(H) for r in range(Sq)]
    ex, rd, ref_lse = oracle.attn_rows(inp.q, inp.k, inp.v, layout, rows, mask=mask, with_lse=True)
    m = MODES.index(mode)
    ex = ex.reshape(B, H, Sq, 128)
    rdm = rd[:, m].reshape(B, H, Sq, 128)
    ref_lse = ref_lse.reshape(B, H, Sq)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    logical = lambda t: np.ascontiguousarray(synth.to_logical(to_bits(t), layout))
    # single pass
    o1 = torch.empty_like(q)
    launch_gqa(q, k, v, o1, layout, mode, mask)
    torch.cuda.synchronize()
    res = gate(logical(o1), rdm, ex)
    assert res.ok, f"single pass: {res.summary()}"
    # the splitting entry point (a split where the plan makes one), with lse
    o2 = torch.empty_like(q)
    lse = torch.full((B, H, Sq), 7.0, dtype=torch.float32, device="cuda:0")
    nbytes = launch_gqa_ws(q, k, v, o2, layout, mode, mask, lse=lse)
    res = gate(logical(o2), rdm, ex)
    assert res.ok, f"split ({nbytes} B workspace): {res.summary()}"
    dmax, nvis = _lse_bound(synth.to_logical(inp.q, layout), synth.to_logical(inp.k, layout), mask, Sq, Sk)
    ok, worst, _ = lse_gate(lse.cpu().numpy(), ref_lse, lse_tolerance(dmax, nvis, ref_lse))
    assert ok, f"lse worst err/tol {worst:.3f}"
    # key shards at a random cut, merged
    rng = np.random.default_rng(5000 + i)
    cuts = sorted({0, Sk, *rng.integers(0, Sk + 1, size=2).tolist()})
    n = len(cuts) - 1
    parts = torch.empty((n,) + tuple(q.shape), dtype=torch.float32, device="cuda:0")
    lses = torch.empty((n, B, H, Sq), dtype=torch.float32, device="cuda:0")
    s = torch.cuda.current_stream().cuda_stream
    keep = []
    for p in range(n):
        k0, k1 = cuts[p], cuts[p + 1]
        if k1 == k0:
            continue
        sl = (lambda t: t[:, k0:k1]) if layout == "bshd" else (lambda t: t[:, :, k0:k1])
        ks, vs = sl(k).contiguous(), sl(v).contiguous()
        keep += [ks, vs]
        st = attn.attn_fwd_bf16_partial(q.data_ptr(), ks.data_ptr(), vs.data_ptr(), parts[p].data_ptr(),
                                        lses[p].data_ptr(), B, H, H_kv, Sq, k1 - k0, k0, Sk, attn.LAYOUTS[layout],
                                        attn.MASKS[mask], s)
        assert st == 0, attn.attn_fwd_bf16_strerror(st)
    torch.cuda.synchronize()
    o3 = torch.empty_like(q)
    st = attn.attn_fwd_bf16_merge(parts.data_ptr(), lses.data_ptr(), n, o3.data_ptr(), 0, B, H, Sq,
                                  attn.LAYOUTS[layout], attn.ROUND_MODES[mode], s)
    assert st == 0
    torch.cuda.synchronize()
    res = gate(logical(o3), rdm, ex)
    assert res.ok, f"shards {cuts}: {res.summary()}"


@pytest.mark.parametrize("i", range(40))
def test_random_varlen_case(i):
    # packed sequences of random lengths (some without queries or without keys), grouped heads,
    # a random mask and mode, through attn_fwd_bf16_varlen with lse
    rng = np.random.default_rng(9000 + i)
    nseq = int(rng.integers(1, 7))
    lq = [int(x) for x in rng.choice([0, 1, 5, 64, 65, 200, 256, 257, 600], size=nseq)]
    lk = [int(x) for x in rng.choice([0, 1, 7, 64, 100, 300, 513, 900], size=nseq)]
    if sum(lq) == 0:
        lq[0] = 3
    if sum(lk) == 0:
        lk[-1] = 5
    H_kv = int(rng.choice([1, 2]))
    H = H_kv * int(rng.choice([1, 3]))
    mode = MODES[rng.integers(3)]
    mask = ["none", "causal", "causal_br"][rng.integers(3)]
    say(f"  varlen case {i}: lq={lq} lk={lk} H={H} H_kv={H_kv} {mode} {mask}")
    wl = synth.VarlenWorkload(f"rv{i}", tuple(lq), tuple(lk), H, H_kv, (mode,), mask=mask, seed=300 + i)
    inp = synth.generate_varlen(wl)
    rows = [(t, h) for t in range(sum(lq)) for h in range(H)]
    ex, rd, ref_lse = oracle.attn_rows_varlen(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, rows, mask=mask,
                                              with_lse=True)
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    k = torch.from_numpy(inp.k.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    v = torch.from_numpy(inp.v.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    cq = torch.from_numpy(inp.cu_q).to("cuda:0")
    ck = torch.from_numpy(inp.cu_k).to("cuda:0")
    out, lse = attn.attn_fwd_varlen(q, k, v, cq, ck, max(lq), round_mode=mode, mask=mask, with_lse=True)
    torch.cuda.synchronize()
    got = to_bits(out).reshape(-1, 128)
    res = gate(got, rd[:, MODES.index(mode)], ex)
    assert res.ok, res.summary()
    got_lse = lse.cpu().numpy().T.reshape(-1)  # [H, total_q] -> rows (t, h)
    # the derived fp32 bound, from each row's own sequence: largest |q|.|k| over its visible keys
    dmax = np.zeros(len(rows))
    nvis = np.zeros(len(rows))
    for b in range(nseq):
        q0, q1, k0, k1 = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        if q1 == q0:
            continue
        qa = np.abs(cases.val(inp.q[q0:q1]))                                   # [Sq, H, 128]
        ka = np.repeat(np.abs(cases.val(inp.k[k0:k1])), H // H_kv, axis=1)   # [Sk, H, 128]
        dots = np.einsum("ihd,jhd->ihj", qa, ka) / math.sqrt(128)
        Sq_b, Sk_b = q1 - q0, k1 - k0
        ii, jj = np.arange(Sq_b)[:, None], np.arange(Sk_b)[None, :]
        vis = np.ones((Sq_b, Sk_b), bool) if mask == "none" else jj <= ii + (0 if mask == "causal" else Sk_b - Sq_b)
        d = np.where(vis[:, None, :], dots, 0.0)
        dmax[q0 * H:q1 * H] = d.max(axis=-1, initial=0.0).reshape(-1)
        nvis[q0 * H:q1 * H] = np.repeat(vis.sum(axis=-1), H)
    ok, worst, _ = lse_gate(got_lse, ref_lse, lse_tolerance(dmax, nvis, ref_lse))
    assert ok, f"lse worst err/tol {worst:.3f}"
