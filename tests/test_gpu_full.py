"""GPU parity at the full workload sizes, in the launch configurations the
benchmark times (one call over the whole tensor: the single pass, and the
key-range split where the shape splits).

The oracle computes sampled rows one by one: seeded random rows of every
head, plus the rows that sit on tile boundaries and at the ragged end of the
query range.  Properties that hold at any size are checked on every row:
repeated launches give identical bits, and in the stressed workload the NaN
rows are exactly the ones the injected K specials must poison.

Then every row of the self-attention (B=4 H=16 8192x8192), cross-attention
(B=2 H=24 4097x32771) and stressed (B=1 H=40 32760x32760) workloads is
compared with the oracle, in chunks of heads (each chunk a test of its own, so
progress shows), every launch configuration the sampled test ran.  On the
inputs drawn N(0,1) the RMS guard of tests/gate.py holds as well.
"""
import time

import numpy as np
import pytest
import torch

import bf16_forward_attention_amd as attn
import oracle
from bf16_forward_attention_amd import synth
from tests.gate import gate, merge
from tests.gpu_util import MODES, Dev, say

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


def _rows_for(wl, n_random=512):
    """Seeded sample plus boundary rows of a few heads."""
    if wl.checked_rows_per_head:
        rows = set(synth.checked_rows(wl))
    else:
        total = wl.B * wl.H * wl.Sq
        flat = synth.floyd_sample(wl.seed, synth.TID_SUBSET, total, min(n_random, total), stream=999)
        rows = {(f // (wl.H * wl.Sq), (f // wl.Sq) % wl.H, f % wl.Sq) for f in flat}
    edge = [0, 1, 63, 64, 127, 128, 255, 256, 257, wl.Sq - 257, wl.Sq - 256, wl.Sq - 2, wl.Sq - 1]
    for bh in (0, wl.B * wl.H - 1, (wl.B * wl.H) // 2):
        for i in edge:
            if 0 <= i < wl.Sq:
                rows.add((bh // wl.H, bh % wl.H, i))
    return sorted(rows)


def _gather(out_stored, layout, rows):
    logical = synth.to_logical(out_stored, layout)
    return np.stack([logical[b, h, i] for b, h, i in rows])


# outputs of the full-size launches, kept for the every-row tests of the same workload:
# name -> (wl, inputs, {(entry, mode): stored output bits})
_OUTPUTS = {}


def _standard_normal(wl) -> bool:
    return wl.qk_sigma == 1.0 and wl.v_dist == "normal" and not wl.scaled_row_fraction and not wl.inject_k_specials


def _run_config(name):
    wl = synth.WORKLOADS[name]
    t0 = time.perf_counter()
    inp = synth.generate(wl)
    say(f"  generated {name} in {time.perf_counter() - t0:.1f} s")
    rows = set(_rows_for(wl))
    for f in inp.scaled_rows[:64]:  # rows of Q scaled by 64
        rows.add((f // (wl.H * wl.Sq), (f // wl.Sq) % wl.H, f % wl.Sq))
    for _, b, h, _, _ in inp.specials:  # rows of the heads with K specials
        for i in synth.floyd_sample(wl.seed, synth.TID_SUBSET, wl.Sq, 32, stream=2000 + b * wl.H + h):
            rows.add((b, h, i))
    rows = sorted(rows)
    t0 = time.perf_counter()
    ex, rd = oracle.attn_rows(inp.q, inp.k, inp.v, wl.layout, rows, mask=wl.mask)
    say(f"  oracle on {len(rows)} rows in {time.perf_counter() - t0:.1f} s")
    dev = Dev(inp)
    outs = {}
    for mode in wl.modes:
        out = dev.run(mode)
        res = gate(_gather(out, wl.layout, rows), rd[:, MODES.index(mode)], ex)
        say(f"  {name} {mode}: {res.summary()}")
        assert res.ok, f"{name} {mode}: {res.summary()}"
        if _standard_normal(wl):
            assert res.rms_guard_ok, f"{name} {mode}: RMS guard: {res.summary()}"
        outs[("single", mode)] = out
    # determinism over the whole tensor
    again = dev.run(wl.modes[0])
    assert np.array_equal(again, outs[("single", wl.modes[0])]), "repeated launch changed the output"
    # the key-range-splitting entry point, where this shape splits (the call the benchmark times then)
    if wl.mask == "none" and wl.kv_heads == wl.H:
        split_bytes = attn.attn_fwd_bf16_workspace_size(wl.B, wl.H, wl.Sq, wl.Sk)
    else:
        split_bytes = attn.attn_fwd_bf16_gqa_workspace_size(wl.B, wl.H, wl.Sq, wl.Sk, attn.MASKS[wl.mask])
    if split_bytes > 0:
        for mode in wl.modes:
            out = dev.run(mode, split=True)
            res = gate(_gather(out, wl.layout, rows), rd[:, MODES.index(mode)], ex)
            say(f"  {name} {mode} split: {res.summary()}")
            assert res.ok, f"{name} {mode} split: {res.summary()}"
            if _standard_normal(wl):
                assert res.rms_guard_ok, f"{name} {mode} split: RMS guard: {res.summary()}"
            outs[("split", mode)] = out
        assert np.array_equal(out, dev.run(wl.modes[-1], split=True)), "split launch not deterministic"
    _OUTPUTS[name] = (wl, inp, outs)
    return wl, inp, {mode: outs[("single", mode)] for mode in wl.modes}


N_CHUNKS = {"self8k": 4, "cross_odd": 4, "dit_stress": 8}


def _every_row_chunk(name, chunk):
    """Compare every row of a chunk of heads with the oracle, for every stored launch."""
    if name not in _OUTPUTS:
        _run_config(name)
    wl, inp, outs = _OUTPUTS[name]
    n_heads = wl.B * wl.H
    heads = range(chunk * n_heads // N_CHUNKS[name], (chunk + 1) * n_heads // N_CHUNKS[name])
    results = {key: [] for key in outs}
    t0 = time.perf_counter()
    logical = {key: synth.to_logical(out, wl.layout) for key, out in outs.items()}
    for bh in heads:
        b, h = divmod(bh, wl.H)
        rows = [(b, h, i) for i in range(wl.Sq)]
        ex, rd = oracle.attn_rows(inp.q, inp.k, inp.v, wl.layout, rows, mask=wl.mask)
        for (entry, mode), lg in logical.items():
            results[(entry, mode)].append(gate(lg[b, h], rd[:, MODES.index(mode)], ex))
    say(f"  {name} heads {heads.start}..{heads.stop - 1}: oracle and gate in {time.perf_counter() - t0:.1f} s")
    for key, parts in results.items():
        res = merge(parts)
        say(f"  {name} {key[0]} {key[1]} every row of heads {heads.start}..{heads.stop - 1}: {res.summary()}")
        assert res.n > 0
        assert res.ok, f"{name} {key}: {res.summary()}"
        if _standard_normal(wl):
            assert res.rms_guard_ok, f"{name} {key}: RMS guard: {res.summary()}"
    if chunk == N_CHUNKS[name] - 1:
        del _OUTPUTS[name]


@pytest.mark.timeout(600)
def test_self_attention_8k():
    # B=4 H=16 Sq=Sk=8192 BSHD RTNE, the benchmarked workload
    _run_config("self8k")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("chunk", range(N_CHUNKS["self8k"]))
def test_self_attention_8k_every_row(chunk):
    # all 524,288 rows, 16 heads per chunk
    _every_row_chunk("self8k", chunk)


@pytest.mark.timeout(600)
def test_cross_attention_odd_lengths():
    # B=2 H=24 Sq=4097 Sk=32771 BSHD RTZ: ragged q-tile and ragged last key tile
    _run_config("cross_odd")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("chunk", range(N_CHUNKS["cross_odd"]))
def test_cross_attention_odd_lengths_every_row(chunk):
    # all 196,656 rows of the single pass and of the key-range split (the launch the benchmark times)
    _every_row_chunk("cross_odd", chunk)


@pytest.mark.timeout(900)
def test_long_context_128k_all_modes():
    # B=1 H=8 Sq=Sk=131072 BHSD, 512 seeded rows per head, every rounding mode
    _run_config("long128k")


@pytest.mark.timeout(900)
def test_stressed_logits_with_k_specials():
    # B=1 H=40 Sq=Sk=32760 BSHD RTNA, Q/K ~ N(0,4), V ~ U(-1,1), 0.1% of Q rows x64,
    # one NaN, one +Inf and one -Inf injected into K
    wl, inp, outs = _run_config("dit_stress")
    out = synth.to_logical(outs["rtna"], wl.layout)
    q = synth.to_logical(inp.q, wl.layout)
    nan_rows = np.all((out & 0x7FFF) > 0x7F80, axis=-1)  # [B, H, Sq]
    any_nan = np.any((out & 0x7FFF) > 0x7F80, axis=-1)
    assert np.array_equal(nan_rows, any_nan), "a row is partly NaN"
    expect = np.zeros_like(nan_rows)
    for bits, b, h, j, c in inp.specials:
        qc = (q[b, h, :, c].astype(np.uint32) << np.uint32(16)).view(np.float32)
        if bits == synth.BF16_NAN:
            expect[b, h, :] = True  # a NaN logit in every row of the head
        elif bits == synth.BF16_PINF:
            expect[b, h, :] = qc >= 0  # +Inf logit (or 0*Inf = NaN) -> NaN row; -Inf drops the key
        else:
            expect[b, h, :] = qc <= 0
    assert np.array_equal(nan_rows, expect), (
        f"NaN rows differ from the rule at {np.argwhere(nan_rows != expect)[:5].tolist()}")
    assert not np.any(((out & 0x7FFF) == 0x7F80)), "an output element is infinite"
    # the x64-scaled rows were sampled too: make sure some were checked
    say(f"  NaN rows: {int(nan_rows.sum())} of {nan_rows.size}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("chunk", range(N_CHUNKS["dit_stress"]))
def test_stressed_logits_every_row(chunk):
    # all 1,310,400 rows (5 heads per chunk): every x64-scaled row, every row of the three heads with
    # a K special, and the rest
    _every_row_chunk("dit_stress", chunk)


@pytest.mark.timeout(600)
def test_causal_self_attention_8k():
    # B=4 H=16 Sq=Sk=8192 BSHD RTNE, diagonal at the top left
    _run_config("self8k_causal")


@pytest.mark.timeout(600)
def test_causal_bottom_right_prefill_odd_lengths():
    # B=2 H=24 Sq=4097 Sk=32771 BSHD RTZ, diagonal at the bottom right: row i sees keys <= i + 28674
    _run_config("prefill_br")


@pytest.mark.timeout(600)
def test_causal_long_sequence_few_heads():
    # B=1 H=4 Sq=Sk=16384 BSHD RTNE, causal: one round of unequal items, all cut into key ranges
    _run_config("causal16k_4h")


@pytest.mark.timeout(600)
def test_grouped_query_causal_8k():
    # B=2 H=32 H_kv=8 Sq=Sk=8192 BSHD RTNE, causal: query head h uses K/V head h / 4
    _run_config("gqa8k_causal")


@pytest.mark.timeout(600)
def test_varlen_mix_causal():
    # 16 packed causal sequences of 732 .. 7793 tokens (77048 in all), H=32 over H_kv=8, RTNE:
    # seeded rows plus the first and last rows of every sequence, checked one by one
    from tests.gpu_util import to_bits, to_device

    wl = synth.VARLEN_WORKLOADS["varlen_mix"]
    inp = synth.generate_varlen(wl)
    total_q = inp.q.shape[0]
    flat = synth.floyd_sample(wl.seed, synth.TID_SUBSET, total_q * wl.H, 768, stream=4242)
    rows = {(f // wl.H, f % wl.H) for f in flat}
    for b in range(wl.B):
        for t in (inp.cu_q[b], inp.cu_q[b] + 255, inp.cu_q[b] + 256, inp.cu_q[b + 1] - 1):
            if inp.cu_q[b] <= t < inp.cu_q[b + 1]:
                rows.add((int(t), (3 * b) % wl.H))
    rows = sorted(rows)
    ex, rd = oracle.attn_rows_varlen(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, rows, wl.mask)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    cq, ck = torch.from_numpy(inp.cu_q).to("cuda:0"), torch.from_numpy(inp.cu_k).to("cuda:0")
    o = torch.empty_like(q)
    outs = []
    for _ in range(2):
        st = attn.attn_fwd_bf16_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), 0, cq.data_ptr(),
                                       ck.data_ptr(), wl.B, wl.H, wl.H_kv, total_q, inp.k.shape[0],
                                       max(wl.lengths_q), attn.ROUND_MODES["rtne"], attn.MASKS[wl.mask],
                                       torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        outs.append(to_bits(o))
    assert np.array_equal(outs[0], outs[1]), "repeated launch changed the output"
    got = np.stack([outs[0][t, h] for t, h in rows])
    res = gate(got, rd[:, 0], ex)
    say(f"  varlen_mix rtne: {res.summary()}")
    assert res.ok, res.summary()


@pytest.mark.timeout(600)
def test_zero_keys_and_values_give_exact_zeros():
    # self8k's shapes and Q with K = V = +0 (the bench's power reference): every logit is 0 and
    # every output a mean of zero rows, +0 in every mode by the definition. Every element of the
    # unmasked, causal and split outputs must be +0, and sampled rows must match the oracle's bits.
    wl = synth.WORKLOADS["self8k_zero_kv"]
    inp = synth.generate(wl)
    rows = _rows_for(wl, n_random=64)
    ex, rd = oracle.attn_rows(inp.q, inp.k, inp.v, wl.layout, rows, mask="none")
    assert not np.any(rd) and not np.any(ex)
    dev = Dev(inp)
    for mode in MODES:
        for kind, out in (("single", dev.run(mode)), ("causal", dev.run(mode, mask="causal")),
                          ("split", dev.run(mode, split=True))):
            nonzero = int(np.count_nonzero(out))
            say(f"  self8k_zero_kv {mode} {kind}: {nonzero} nonzero elements")
            assert nonzero == 0, f"{mode} {kind}: {nonzero} elements are not +0"
            res = gate(_gather(out, wl.layout, rows), rd[:, MODES.index(mode)], ex)
            assert res.ok and res.max_row_ulps == 0, f"{mode} {kind}: {res.summary()}"
