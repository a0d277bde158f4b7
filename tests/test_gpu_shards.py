"""GPU parity of key sharding: attn_fwd_bf16_partial on each shard of the
keys, then attn_fwd_bf16_merge, against the fp64 oracle of the whole problem.

The keys of each head are cut into consecutive shards (ragged cuts, causal
diagonals crossing them, shards that some rows see nothing of), each shard
is run on its own K/V slice, and the merge must give every row within the
row-scaled 2-ULP gate in every rounding mode and the whole row's
log-sum-exp within its fp32 bound.  One shard over all keys must give
exactly the single-pass bits (the partial row is the single pass's fp32 row
and its merge weight is exactly 1).
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
from tests.gpu_util import MODES, launch_gqa, say, to_bits, to_device

pytestmark = pytest.mark.gpu

U = 2.0**-24


@pytest.fixture(autouse=True)
def _name_the_case(request):
    say(f"[gpu case] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield


def _dims(q, k, layout):
    if layout == "bshd":
        return q.shape[0], q.shape[2], k.shape[2], q.shape[1], k.shape[1]
    return q.shape[0], q.shape[1], k.shape[1], q.shape[2], k.shape[2]


def _shard(t, layout, s0, s1):
    return (t[:, s0:s1] if layout == "bshd" else t[:, :, s0:s1]).contiguous()


def run_shards(q, k, v, layout, mask, cuts):
    """Partials of the shards [cuts[i], cuts[i+1]) of the keys: (o_parts, lse_parts)."""
    B, H, H_kv, Sq, Sk_total = _dims(q, k, layout)
    n = len(cuts) - 1
    o_parts = torch.full((n,) + tuple(q.shape), 7.0, dtype=torch.float32, device=q.device)
    lse_parts = torch.full((n, B, H, Sq), 7.0, dtype=torch.float32, device=q.device)
    s = torch.cuda.current_stream().cuda_stream
    keep = []
    for i in range(n):
        ks, vs = _shard(k, layout, cuts[i], cuts[i + 1]), _shard(v, layout, cuts[i], cuts[i + 1])
        keep += [ks, vs]
        st = attn.attn_fwd_bf16_partial(q.data_ptr(), ks.data_ptr(), vs.data_ptr(), o_parts[i].data_ptr(),
                                        lse_parts[i].data_ptr(), B, H, H_kv, Sq, cuts[i + 1] - cuts[i], cuts[i],
                                        Sk_total, attn.LAYOUTS[layout], attn.MASKS[mask], s)
        assert st == 0, attn.attn_fwd_bf16_strerror(st)
    torch.cuda.synchronize()
    return o_parts, lse_parts


def merge(o_parts, lse_parts, q, layout, mode, with_lse=True):
    B, H, _, Sq, _ = _dims(q, q, layout)
    o = torch.empty_like(q)
    lse = torch.full((B, H, Sq), 7.0, dtype=torch.float32, device=q.device) if with_lse else None
    st = attn.attn_fwd_bf16_merge(o_parts.data_ptr(), lse_parts.data_ptr(), o_parts.shape[0], o.data_ptr(),
                                  lse.data_ptr() if with_lse else 0, B, H, Sq, attn.LAYOUTS[layout],
                                  attn.ROUND_MODES[mode], torch.cuda.current_stream().cuda_stream)
    assert st == 0, attn.attn_fwd_bf16_strerror(st)
    torch.cuda.synchronize()
    return o, lse


def _lse_inputs(q_log, k_log, mask, Sq, Sk):
    H, H_kv = q_log.shape[1], k_log.shape[1]
    qa = np.abs(cases.val(q_log))
    ka = np.repeat(np.abs(cases.val(k_log)), H // H_kv, axis=1)
    dots = np.einsum("bhid,bhjd->bhij", qa, ka) / math.sqrt(128)
    i, j = np.arange(Sq)[:, None], np.arange(Sk)[None, :]
    vis = np.ones((Sq, Sk), bool) if mask == "none" else j <= i + (0 if mask == "causal" else Sk - Sq)
    dots = np.where(vis, dots, 0.0)
    return dots.max(axis=-1, initial=0.0), np.broadcast_to(vis.sum(axis=-1), dots.shape[:-1])


# (B, H, H_kv, Sq, Sk_total, cuts)
SHAPES = [
    (1, 4, 2, 300, 1000, [0, 257, 600, 1000]),
    (2, 2, 2, 700, 700, [0, 64, 65, 700]),            # a one-key shard
    (1, 2, 1, 500, 300, [0, 100, 300]),               # Sq > Sk: bottom-right rows without any key
    (1, 3, 3, 129, 4000, [0, 1000, 2000, 3000, 4000]),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:5])) + f"_{len(s[5]) - 1}shards")
@pytest.mark.parametrize("mask", ["none", "causal", "causal_br"])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_merged_shards_match_the_oracle(shape, mask, layout):
    B, H, H_kv, Sq, Sk, cuts = shape
    inp = synth.small(B, H, Sq, Sk, layout, seed=Sq + Sk + len(cuts), qk_sigma=1.5, mask=mask, H_kv=H_kv)
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(Sq)]
    ex, rd, ref_lse = oracle.attn_rows(inp.q, inp.k, inp.v, layout, rows, mask=mask, with_lse=True)
    ex = ex.reshape(B, H, Sq, 128)
    rd = np.moveaxis(rd.reshape(B, H, Sq, 3, 128), 3, 0)
    ref_lse = ref_lse.reshape(B, H, Sq)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    o_parts, lse_parts = run_shards(q, k, v, layout, mask, cuts)
    n = len(cuts) - 1
    for m, mode in enumerate(MODES):
        o, lse = merge(o_parts, lse_parts, q, layout, mode)
        got = np.ascontiguousarray(synth.to_logical(to_bits(o), layout))
        res = gate(got, rd[m], ex)
        say(f"  {shape[:5]} {mask} {layout} {mode}: {res.summary()}")
        assert res.ok, res.summary()
        if m == 0:
            dmax, nvis = _lse_inputs(synth.to_logical(inp.q, layout), synth.to_logical(inp.k, layout), mask, Sq, Sk)
            # the merge adds one exp and one product per shard and a final log and add to the
            # fp32 errors lse_tolerance bounds for the whole row
            tol = lse_tolerance(dmax, nvis, ref_lse) + (16 * U) * (1 + np.abs(ref_lse)) + 4 * n * U
            ok, worst, cnt = lse_gate(lse.cpu().numpy(), ref_lse, tol)
            say(f"  merged lse worst err/tol {worst:.3f} over {cnt} rows")
            assert ok, f"merged lse worst err/tol {worst:.3f}"
    again = merge(*run_shards(q, k, v, layout, mask, cuts), q, layout, MODES[0], with_lse=False)[0]
    assert np.array_equal(to_bits(again), to_bits(merge(o_parts, lse_parts, q, layout, MODES[0])[0]))


@pytest.mark.parametrize("mask", ["none", "causal", "causal_br"])
def test_rows_that_see_no_key_of_a_shard(mask):
    # top left: the rows before a shard's first key see none of it; bottom right with
    # Sq > Sk: the first Sq - Sk rows see no key at all
    B, H, Sq, Sk, cuts = 1, 2, 400, 300, [0, 150, 300]
    inp = synth.small(B, H, Sq, Sk, "bshd", seed=9, mask=mask)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    o_parts, lse_parts = run_shards(q, k, v, "bshd", mask, cuts)
    off = {"none": None, "causal": 0, "causal_br": Sk - Sq}[mask]
    lp = lse_parts.cpu().numpy()
    op = o_parts.cpu().numpy()  # [n, B, Sq, H, 128]
    for s in range(2):
        for i in range(Sq):
            sees = off is None or i + off >= cuts[s]
            if sees:
                assert np.all(np.isfinite(lp[s, :, :, i])), (s, i)
            else:
                assert np.all(lp[s, :, :, i] == -np.inf), (s, i)
                assert np.all(op[s, :, i] == 0.0), (s, i)
    o, lse = merge(o_parts, lse_parts, q, "bshd", "rtne")
    got = synth.to_logical(to_bits(o), "bshd")
    empty = np.array([off is not None and i + off < 0 for i in range(Sq)])
    assert np.all(lse.cpu().numpy()[:, :, empty] == -np.inf)
    assert np.all((got[:, :, empty] & 0x7FFF) > 0x7F80), "a row without keys must be NaN"
    assert np.all(np.isfinite(lse.cpu().numpy()[:, :, ~empty]))


@pytest.mark.parametrize("mask", ["none", "causal", "causal_br"])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_one_shard_is_the_single_pass(mask, layout):
    B, H, H_kv, Sq, Sk = 2, 4, 2, 333, 517
    inp = synth.small(B, H, Sq, Sk, layout, seed=12, mask=mask, H_kv=H_kv)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    o_parts, lse_parts = run_shards(q, k, v, layout, mask, [0, Sk])
    for mode in MODES:
        o, lse = merge(o_parts, lse_parts, q, layout, mode)
        o1 = torch.empty_like(q)
        lse1 = torch.empty_like(lse)
        launch_gqa(q, k, v, o1, layout, mode, mask, lse=lse1)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(o), to_bits(o1)), mode
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), lse1.cpu().numpy().view(np.uint32)), mode


def test_nan_and_inf_keys_through_the_merge():
    # R1-R3: a NaN key element makes every row of its head NaN; an infinite one makes the rows
    # whose logit becomes +Inf (or 0 * Inf) NaN and drops the key from the rest: positions as
    # the oracle's
    B, H, Sq, Sk, cuts = 1, 3, 200, 600, [0, 200, 400, 600]
    inp = synth.small(B, H, Sq, Sk, "bhsd", seed=31)
    k = inp.k.copy()
    k[0, 0, 250, 5] = 0x7FC0   # NaN in the second shard of head 0
    k[0, 1, 450, 7] = 0x7F80   # +Inf in the third shard of head 1
    k[0, 2, 10, 9] = 0xFF80    # -Inf in the first shard of head 2
    ex, rd = oracle.attn_all(inp.q, k, inp.v, "bhsd")
    q, kk, v = to_device(inp.q), to_device(k), to_device(inp.v)
    o_parts, lse_parts = run_shards(q, kk, v, "bhsd", "none", cuts)
    o, lse = merge(o_parts, lse_parts, q, "bhsd", "rtna")
    got = np.ascontiguousarray(to_bits(o))
    res = gate(got, rd[1], ex)
    say(f"  specials: {res.summary()}")
    assert res.ok, res.summary()
    nan_rows = np.all(np.isnan(ex), axis=-1)
    # head 0: every row; heads 1 and 2: the rows whose q entry makes the logit +Inf (or 0 * Inf)
    assert nan_rows[0, 0].all() and nan_rows[0, 1].any() and not nan_rows[0, 1].all()
    assert nan_rows[0, 2].any() and not nan_rows[0, 2].all()
    assert np.array_equal(np.isnan(lse.cpu().numpy()), nan_rows)


def test_shards_far_along_a_long_sequence():
    # A shard of 1000 keys at the end of a sequence of 2^31 - 1 keys (only the shard is allocated):
    # with the top-left diagonal no row of a short query block sees any of its keys (the offset
    # from the diagonal is about -2^31: 0 rows and an lse of -Inf); with the bottom-right one the
    # last shard sees exactly what a bottom-right call on the shard alone sees, so its single-shard
    # merge gives that call's bits.
    B, H, Sq, Sk = 1, 2, 300, 1000
    total = (1 << 31) - 1
    inp = synth.small(B, H, Sq, Sk, "bshd", seed=44)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    s = torch.cuda.current_stream().cuda_stream
    for mask in ("causal", "causal_br"):
        o_part = torch.full((1,) + tuple(q.shape), 7.0, dtype=torch.float32, device="cuda:0")
        lse_part = torch.full((1, B, H, Sq), 7.0, dtype=torch.float32, device="cuda:0")
        st = attn.attn_fwd_bf16_partial(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_part.data_ptr(),
                                        lse_part.data_ptr(), B, H, H, Sq, Sk, total - Sk, total,
                                        attn.LAYOUTS["bshd"], attn.MASKS[mask], s)
        assert st == 0, attn.attn_fwd_bf16_strerror(st)
        torch.cuda.synchronize()
        if mask == "causal":
            assert np.all(lse_part.cpu().numpy() == -np.inf)
            assert np.all(o_part.cpu().numpy() == 0.0)
        else:
            o, lse = merge(o_part, lse_part, q, "bshd", "rtna")
            o1, lse1 = torch.empty_like(q), torch.empty_like(lse)
            launch_gqa(q, k, v, o1, "bshd", "rtna", "causal_br", lse=lse1)
            torch.cuda.synchronize()
            assert np.array_equal(to_bits(o), to_bits(o1))
            assert np.array_equal(lse.cpu().numpy().view(np.uint32), lse1.cpu().numpy().view(np.uint32))


def test_partial_and_merge_write_only_their_rows():
    B, H, Sq, Sk, cuts = 1, 2, 300, 700, [0, 300, 700]
    inp = synth.small(B, H, Sq, Sk, "bhsd", seed=62)
    q, k, v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
    pad, n_rows = 4096, B * H * Sq
    n_part = q.numel()
    p_buf = torch.full((2 * n_part + 2 * pad,), -777.0, dtype=torch.float32, device="cuda:0")
    l_buf = torch.full((2 * n_rows + 2 * pad,), -777.0, dtype=torch.float32, device="cuda:0")
    o_parts = p_buf[pad:pad + 2 * n_part].view((2,) + tuple(q.shape))
    lse_parts = l_buf[pad:pad + 2 * n_rows].view(2, B, H, Sq)
    s = torch.cuda.current_stream().cuda_stream
    for i in range(2):
        ks, vs = _shard(k, "bhsd", cuts[i], cuts[i + 1]), _shard(v, "bhsd", cuts[i], cuts[i + 1])
        assert attn.attn_fwd_bf16_partial(q.data_ptr(), ks.data_ptr(), vs.data_ptr(), o_parts[i].data_ptr(),
                                          lse_parts[i].data_ptr(), B, H, H, Sq, cuts[i + 1] - cuts[i], cuts[i], Sk,
                                          attn.LAYOUTS["bhsd"], attn.MASKS["none"], s) == 0
        torch.cuda.synchronize()
    o_buf = torch.full((q.numel() + 2 * pad,), 0x7E7E, dtype=torch.int16, device="cuda:0")
    m_buf = torch.full((n_rows + 2 * pad,), -777.0, dtype=torch.float32, device="cuda:0")
    o = o_buf[pad:pad + q.numel()]
    lse = m_buf[pad:pad + n_rows]
    assert attn.attn_fwd_bf16_merge(o_parts.data_ptr(), lse_parts.data_ptr(), 2, o.data_ptr(), lse.data_ptr(), B, H,
                                    Sq, attn.LAYOUTS["bhsd"], attn.ROUND_MODES["rtz"], s) == 0
    torch.cuda.synchronize()
    for buf, n, fill in ((p_buf, 2 * n_part, -777.0), (l_buf, 2 * n_rows, -777.0), (m_buf, n_rows, -777.0)):
        a = buf.cpu().numpy()
        assert np.all(a[:pad] == fill) and np.all(a[pad + n:] == fill)
        assert not np.any(a[pad:pad + n] == fill)  # every element inside was written
    ob = o_buf.cpu().numpy()
    assert np.all(ob[:pad] == 0x7E7E) and np.all(ob[pad + q.numel():] == 0x7E7E)
