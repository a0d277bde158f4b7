"""Hand-built structured inputs shared by the oracle pins and the GPU tests.

Builders return logical [B, H, S, 128] uint16 (bf16 bit) arrays; use
``synth.to_layout`` to store them.  Nothing here computes attention.
"""
from __future__ import annotations

import os

import numpy as np

from bf16_forward_attention_amd import synth

D = 128
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bf(x) -> np.ndarray:
    """bf16 bits of values that are exactly representable in bf16."""
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32)
    if np.any(bits & np.uint32(0xFFFF)):
        raise ValueError("value not representable in bf16")
    return (bits >> np.uint32(16)).astype(np.uint16)


def val(bits) -> np.ndarray:
    """float64 values of bf16 bits (via float32, exact)."""
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def randn_bits(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    return synth.normal_bf16(seed, 7, n, sigma).reshape(shape)


def dominant(B, H, Sq, Sk, seed=0):
    """Inputs where each query row has one dominant key.

    Row i of a head points along direction c_i = 1 + (i mod 127): q[i, c_i] =
    128 and every other entry of q is 0.  Per head and direction one key
    jmap[c] has k[jmap, c] = 128 and every other key has k[., c] = 0.  So the
    logit of that key is 128*128/sqrt(128) ~ 1448 and every other logit is 0:
    exp(-1448) underflows to 0 even in binary64, and O_i = V[jmap[c_i]]
    exactly.  Returns (q, k, v, jstar) with jstar[b, h, i] the dominant key.
    """
    rng = np.random.default_rng(seed)
    q = np.zeros((B, H, Sq, D), np.uint16)
    k = randn_bits((B, H, Sk, D), seed + 1)
    v = randn_bits((B, H, Sk, D), seed + 2)
    jstar = np.zeros((B, H, Sq), np.int64)
    for b in range(B):
        for h in range(H):
            jmap = rng.integers(0, Sk, D)
            # keep the last key in play so tail tiles are exercised
            jmap[1 + (Sq - 1) % (D - 1)] = Sk - 1
            for c in range(1, D):
                k[b, h, :, c] = 0
                k[b, h, jmap[c], c] = bf(128.0)
            for i in range(Sq):
                c = 1 + (i % (D - 1))
                q[b, h, i, c] = bf(128.0)
                jstar[b, h, i] = jmap[c]
    return q, k, v, jstar


def load_ties():
    """Rows of tests/golden/midpoint_ties.txt: (v_bits list, (rtne, rtna, rtz), scope)."""
    rows = []
    with open(os.path.join(GOLDEN, "midpoint_ties.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            vals, rtne, rtna, rtz, scope = line.split()
            rows.append(([int(x, 16) for x in vals.split(",")], (int(rtne, 16), int(rtna, 16), int(rtz, 16)), scope))
    return rows


def tie_inputs(vals):
    """One head, one query, len(vals) keys with equal logits (Q = 0, K = 0):
    every column of V holds ``vals``, so every output element is their mean."""
    n = len(vals)
    q = np.zeros((1, 1, 1, D), np.uint16)
    k = np.zeros((1, 1, n, D), np.uint16)
    v = np.repeat(np.asarray(vals, np.uint16)[:, None], D, axis=1).reshape(1, 1, n, D)
    return q, k, v


def diagonal_dominant(B, H, Sq, Sk, off, seed=0):
    """Inputs where row i's key j = i + off (when 0 <= j < Sk) dominates.

    Needs Sq <= 127: row i points along direction c_i = 1 + i; column c_i of K
    is 0 except k[i + off, c_i] = 128, so that key's logit is ~1448 and every
    other key's is 0 or a random multiple of 128 * k / sqrt(128) far below it
    (K's other columns stay random).  A row whose key lies past the end of K
    has q = 0.  Returns (q, k, v).
    """
    assert Sq <= D - 1
    q = np.zeros((B, H, Sq, D), np.uint16)
    k = randn_bits((B, H, Sk, D), seed + 1)
    v = randn_bits((B, H, Sk, D), seed + 2)
    k[:, :, :, 1:Sq + 1] = 0
    for i in range(Sq):
        j = i + off
        if 0 <= j < Sk:
            q[:, :, i, 1 + i] = bf(128.0)
            k[:, :, j, 1 + i] = bf(128.0)
    return q, k, v


def subnormal_bits(shape, seed: int, tensor_id: int = 9) -> np.ndarray:
    """bf16 subnormals: random sign, significand 1..127 (values k * 2^-133),
    from the seeded counter-based stream."""
    n = int(np.prod(shape))
    u = synth.u64_at(synth.stream_key(seed, tensor_id), np.arange(n, dtype=np.uint64))
    mag = (u % np.uint64(127)).astype(np.uint16) + np.uint16(1)
    sign = ((u >> np.uint64(32)) & np.uint64(1)).astype(np.uint16) << np.uint16(15)
    return (mag | sign).reshape(shape)


def scaled_bits(shape, seed: int, exp_shift: int, tensor_id: int = 10) -> np.ndarray:
    """bf16 values u * 2^exp_shift with u ~ U(-1.9, 1.9) (normal bf16 values of
    that range, zero kept), by adding ``exp_shift`` to the exponent field."""
    n = int(np.prod(shape))
    b = synth.uniform_bf16(seed, tensor_id, n, -1.9, 1.9).astype(np.int32)
    e = (b >> 7) & 0xFF
    if np.any((e != 0) & ((e + exp_shift < 1) | (e + exp_shift > 254))):
        raise ValueError("shift leaves the normal bf16 range")
    out = np.where(e != 0, b + (exp_shift << 7), b)
    return out.astype(np.uint16).reshape(shape)
