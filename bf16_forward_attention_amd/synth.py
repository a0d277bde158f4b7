"""Seeded synthetic inputs for bf16 forward attention (d = 128).

This module only draws input tensors: it holds none of the attention
arithmetic and none of the output rounding. Both the GPU path's tests and
the CPU oracle's tests take their inputs from here, so the two sides see the
same bytes.

Random numbers are counter based, so any element can be drawn on its own:

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014).  State n of a stream seeded with ``key`` is
  ``key + (n + 1) * GAMMA`` (mod 2^64); the output is the 64-bit finaliser
  ``mix64`` of that state.  A tensor's stream key is itself the output of the
  stream seeded with ``seed`` at position ``tensor_id``.
* Normal variates by the Box-Muller transform (Box and Muller, 1958) from the
  two uniforms at counters 2n and 2n+1.
* Values are indexed by their LOGICAL position (b, h, s, c), i.e. by the
  BHSD offset ``((b*H + h)*S + s)*128 + c``; a BSHD tensor is the same
  logical tensor stored in the other order.

Inputs are quantised from float64 to bf16 with round-to-nearest-even on the
float64 bit pattern (an input-preparation step, independent of the output
rounding under test).

Tensor ids: Q = 0, K = 1, V = 2, scaled-row choice = 3, injected specials = 4,
checked-row subset = 5.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

D = 128
GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1

TID_Q, TID_K, TID_V, TID_ROWSCALE, TID_SPECIAL, TID_SUBSET = 0, 1, 2, 3, 4, 5
TID_LENGTHS = 6  # sequence lengths of the variable-length batches

LAYOUTS = ("bshd", "bhsd")
MODES = ("rtne", "rtna", "rtz")

BF16_NAN = 0x7FC0
BF16_PINF = 0x7F80
BF16_NINF = 0xFF80


# --------------------------------------------------------------------------
# SplitMix64, vectorised over counters
# --------------------------------------------------------------------------
def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tensor_id: int) -> int:
    """Key of the stream for one tensor: output ``tensor_id`` of stream ``seed``."""
    return _mix64_int(seed + (tensor_id + 1) * int(GAMMA))


def u64_at(key: int, counters: np.ndarray) -> np.ndarray:
    """SplitMix64 outputs of stream ``key`` at the given counters (uint64)."""
    with np.errstate(over="ignore"):
        st = np.uint64(key) + (counters.astype(np.uint64) + np.uint64(1)) * GAMMA
        return _mix64(st)


def u64_int(key: int, counter: int) -> int:
    return _mix64_int(key + (counter + 1) * int(GAMMA))


# --------------------------------------------------------------------------
# float64 -> bf16 bits (input quantisation only)
# --------------------------------------------------------------------------
def _f64_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Quantise finite float64 values with |x| >= 2^-126 or x == 0 to bf16 bits.

    Rounds the float64 significand to 8 significant bits (ties to even) by
    integer arithmetic on the bit pattern, then reads the exactly
    representable result through float32.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(~np.isfinite(a)) or np.any((a != 0) & (a < 2.0**-126)) or np.any(a >= 2.0**127):
        raise ValueError("generator value outside the normal bf16 range")
    bits = x.view(np.uint64)
    half = np.uint64((1 << 44) - 1)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    r = (bits + half + lsb) & ~np.uint64((1 << 45) - 1)
    f32 = r.view(np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# distributions over a logical index range
# --------------------------------------------------------------------------
def _normal_chunk(key: int, lo: int, hi: int, sigma: float) -> np.ndarray:
    n = np.arange(lo, hi, dtype=np.uint64)
    x1 = u64_at(key, n * np.uint64(2))
    x2 = u64_at(key, n * np.uint64(2) + np.uint64(1))
    u1 = ((x1 >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0**-53  # (0, 1]
    u2 = (x2 >> np.uint64(11)).astype(np.float64) * 2.0**-53  # [0, 1)
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    # Box-Muller can only give |z| < 2^-126 by landing on an exact zero of cos;
    # that value is then flushed to zero.
    z = np.where(np.abs(z) < 2.0**-126, 0.0, z)
    return _f64_to_bf16_rne(z * sigma)


def _uniform_chunk(key: int, lo: int, hi: int, a: float, b: float) -> np.ndarray:
    n = np.arange(lo, hi, dtype=np.uint64)
    u = (u64_at(key, n) >> np.uint64(11)).astype(np.float64) * 2.0**-53  # [0, 1)
    z = a + (b - a) * u
    z = np.where(np.abs(z) < 2.0**-126, 0.0, z)
    return _f64_to_bf16_rne(z)


_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill(fn, key: int, total: int, *args) -> np.ndarray:
    out = np.empty(total, dtype=np.uint16)
    spans = [(lo, min(total, lo + _CHUNK)) for lo in range(0, total, _CHUNK)]

    def work(span):
        lo, hi = span
        out[lo:hi] = fn(key, lo, hi, *args)

    if len(spans) <= 1:
        for s in spans:
            work(s)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, spans))
    return out


def normal_bf16(seed: int, tensor_id: int, total: int, sigma: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0, sigma^2) draws at logical indices 0..total-1."""
    return _fill(_normal_chunk, stream_key(seed, tensor_id), total, sigma)


def uniform_bf16(seed: int, tensor_id: int, total: int, a: float, b: float) -> np.ndarray:
    """bf16 bits of U(a, b) draws at logical indices 0..total-1."""
    return _fill(_uniform_chunk, stream_key(seed, tensor_id), total, a, b)


# --------------------------------------------------------------------------
# sampling without replacement (Floyd), integer arithmetic only
# --------------------------------------------------------------------------
def floyd_sample(seed: int, tensor_id: int, population: int, count: int, stream: int = 0) -> list[int]:
    """``count`` distinct integers in [0, population), sorted.

    Floyd's algorithm (Bentley and Floyd, CACM 1987).  The draw for step j
    is ``(u * (j + 1)) >> 64`` with u the SplitMix64 output at counter
    ``stream * 2^32 + step``.
    """
    if not 0 <= count <= population:
        raise ValueError("count out of range")
    key = stream_key(seed, tensor_id)
    chosen: set[int] = set()
    for step, j in enumerate(range(population - count, population)):
        u = u64_int(key, (stream << 32) + step)
        t = (u * (j + 1)) >> 64
        chosen.add(j if t in chosen else t)
    return sorted(chosen)


# --------------------------------------------------------------------------
# layouts
# --------------------------------------------------------------------------
def to_layout(logical_bhsd: np.ndarray, layout: str) -> np.ndarray:
    """Store a logical [B, H, S, 128] tensor in ``layout`` (a contiguous copy)."""
    if layout == "bhsd":
        return np.ascontiguousarray(logical_bhsd)
    if layout == "bshd":
        return np.ascontiguousarray(logical_bhsd.transpose(0, 2, 1, 3))
    raise ValueError(layout)


def to_logical(stored: np.ndarray, layout: str) -> np.ndarray:
    """View a stored tensor as logical [B, H, S, 128] (no copy)."""
    if layout == "bhsd":
        return stored
    if layout == "bshd":
        return stored.transpose(0, 2, 1, 3)
    raise ValueError(layout)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    layout: str
    modes: tuple
    qk_sigma: float = 1.0
    v_dist: str = "normal"  # "normal" -> N(0,1); "uniform" -> U(-1,1)
    scaled_row_fraction: float = 0.0  # fraction of Q rows multiplied by 64
    inject_k_specials: bool = False  # one NaN, one +Inf, one -Inf in K
    checked_rows_per_head: int = 0  # 0: every row is checkable
    seed: int = 0
    mask: str = "none"  # key mask the workload is run with: "none", "causal", "causal_br"
    H_kv: int = 0  # K/V heads (grouped-query attention); 0: as many as query heads
    zero_kv: bool = False  # K and V all +0 (Q as drawn): same work, operands that barely toggle

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def flops(self) -> int:
        """4 d FLOP per (query, key) pair of the unmasked problem."""
        return 4 * self.B * self.H * self.Sq * self.Sk * D


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 256, 256, "bhsd", MODES),
    "self8k": Workload("self8k", 4, 16, 8192, 8192, "bshd", ("rtne",)),
    "long128k": Workload("long128k", 1, 8, 131072, 131072, "bhsd", MODES, checked_rows_per_head=512),
    "cross_odd": Workload("cross_odd", 2, 24, 4097, 32771, "bshd", ("rtz",)),
    "dit_stress": Workload(
        "dit_stress", 1, 40, 32760, 32760, "bshd", ("rtna",),
        qk_sigma=2.0, v_dist="uniform", scaled_row_fraction=0.001, inject_k_specials=True,
    ),
    # causal self-attention at the benchmark shape, and a chunk of new queries
    # against a longer key cache (diagonal at the bottom right, ragged tiles)
    "self8k_causal": Workload("self8k_causal", 4, 16, 8192, 8192, "bshd", ("rtne",), mask="causal"),
    "prefill_br": Workload("prefill_br", 2, 24, 4097, 32771, "bshd", ("rtz",), mask="causal_br"),
    # grouped-query causal prefill: 32 query heads over 8 K/V heads
    "gqa8k_causal": Workload("gqa8k_causal", 2, 32, 8192, 8192, "bshd", ("rtne",), mask="causal", H_kv=8),
    # one long causal sequence over few heads: 256 work items of 4 .. 256 key tiles, a single round
    "causal16k_4h": Workload("causal16k_4h", 1, 4, 16384, 16384, "bshd", ("rtne",), mask="causal"),
    # a power diagnostic: the self8k shapes and instruction stream with K = V = 0 (every logit 0,
    # every output row exactly 0), so the matrix cores multiply zeros; set against self8k it shows
    # how much of the board power the arithmetic on random data draws
    "self8k_zero_kv": Workload("self8k_zero_kv", 4, 16, 8192, 8192, "bshd", ("rtne",), zero_kv=True),
}


@dataclass
class Inputs:
    wl: Workload
    q: np.ndarray  # uint16 bf16 bits, stored in wl.layout
    k: np.ndarray
    v: np.ndarray
    scaled_rows: list = field(default_factory=list)  # flat logical (b*H + h)*Sq + i
    specials: list = field(default_factory=list)  # (bits, b, h, j, c)


def scaled_row_list(wl: Workload) -> list[int]:
    n_rows = wl.B * wl.H * wl.Sq
    count = int(wl.scaled_row_fraction * n_rows)
    if count == 0:
        return []
    return floyd_sample(wl.seed, TID_ROWSCALE, n_rows, count)


def special_list(wl: Workload) -> list[tuple]:
    """Three K specials (NaN, +Inf, -Inf) in three distinct (b, h) heads."""
    if not wl.inject_k_specials:
        return []
    heads = floyd_sample(wl.seed, TID_SPECIAL, wl.B * wl.kv_heads, 3, stream=0)
    key = stream_key(wl.seed, TID_SPECIAL)
    order = [u64_int(key, (1 << 32) + t) for t in range(3)]
    # shuffle which head gets which special, deterministically
    heads = [h for _, h in sorted(zip(order, heads))]
    out = []
    for t, (bits, bh) in enumerate(zip((BF16_NAN, BF16_PINF, BF16_NINF), heads)):
        j = (u64_int(key, (2 << 32) + t) * wl.Sk) >> 64
        c = (u64_int(key, (3 << 32) + t) * D) >> 64
        out.append((bits, bh // wl.kv_heads, bh % wl.kv_heads, int(j), int(c)))
    return out


def checked_rows(wl: Workload) -> list[tuple]:
    """(b, h, i) rows the oracle checks at full size for ``wl``.

    With ``checked_rows_per_head`` set: that many distinct rows per head
    (Floyd, one sub-stream per head). Otherwise every row.
    """
    rows = []
    for b in range(wl.B):
        for h in range(wl.H):
            if wl.checked_rows_per_head:
                idx = floyd_sample(wl.seed, TID_SUBSET, wl.Sq, wl.checked_rows_per_head, stream=b * wl.H + h)
            else:
                idx = range(wl.Sq)
            rows.extend((b, h, i) for i in idx)
    return rows


def generate(wl: Workload) -> Inputs:
    """Draw Q, K, V for ``wl`` and store them in ``wl.layout``."""
    nq = wl.B * wl.H * wl.Sq * D
    nk = wl.B * wl.kv_heads * wl.Sk * D
    q = normal_bf16(wl.seed, TID_Q, nq, wl.qk_sigma).reshape(wl.B, wl.H, wl.Sq, D)
    if wl.zero_kv:
        k = np.zeros((wl.B, wl.kv_heads, wl.Sk, D), dtype=np.uint16)
        v = np.zeros((wl.B, wl.kv_heads, wl.Sk, D), dtype=np.uint16)
        return Inputs(wl, to_layout(q, wl.layout), to_layout(k, wl.layout), to_layout(v, wl.layout), [], [])
    k = normal_bf16(wl.seed, TID_K, nk, wl.qk_sigma).reshape(wl.B, wl.kv_heads, wl.Sk, D)
    if wl.v_dist == "normal":
        v = normal_bf16(wl.seed, TID_V, nk, 1.0)
    elif wl.v_dist == "uniform":
        v = uniform_bf16(wl.seed, TID_V, nk, -1.0, 1.0)
    else:
        raise ValueError(wl.v_dist)
    v = v.reshape(wl.B, wl.kv_heads, wl.Sk, D)

    rows = scaled_row_list(wl)
    if rows:
        flat = q.reshape(-1, D)
        # x64 is a power of two: exact in float32, and the product keeps a
        # bf16 significand, so taking the top 16 bits is exact.
        f = (flat[rows].astype(np.uint32) << np.uint32(16)).view(np.float32) * np.float32(64.0)
        if not np.all(np.isfinite(f)) or np.any(np.abs(f) >= 2.0**127):
            raise ValueError("row scaling would leave the bf16 range")
        flat[rows] = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    specials = special_list(wl)
    for bits, b, h, j, c in specials:
        k[b, h, j, c] = bits
    return Inputs(wl, to_layout(q, wl.layout), to_layout(k, wl.layout), to_layout(v, wl.layout), rows, specials)


def small(B: int, H: int, Sq: int, Sk: int, layout: str = "bshd", seed: int = 0,
          qk_sigma: float = 1.0, v_dist: str = "normal", mask: str = "none", H_kv: int = 0) -> Inputs:
    """A small i.i.d. workload for parity tests."""
    wl = Workload(f"small_{B}x{H}x{H_kv or H}x{Sq}x{Sk}_{layout}_{mask}", B, H, Sq, Sk, layout, MODES,
                  qk_sigma=qk_sigma, v_dist=v_dist, seed=seed, mask=mask, H_kv=H_kv)
    return generate(wl)


# --------------------------------------------------------------------------
# variable-length batches (sequences packed one after another)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class VarlenWorkload:
    name: str
    lengths_q: tuple  # query rows of each sequence
    lengths_k: tuple  # key rows of each sequence
    H: int
    H_kv: int
    modes: tuple
    mask: str = "none"
    seed: int = 0

    @property
    def B(self) -> int:
        return len(self.lengths_q)


@dataclass
class VarlenInputs:
    wl: VarlenWorkload
    q: np.ndarray  # uint16 bf16 bits [total_q, H, 128]
    k: np.ndarray  # [total_k, H_kv, 128]
    v: np.ndarray
    cu_q: np.ndarray  # int32 [B + 1]: sequence b holds packed rows cu[b] .. cu[b+1]-1
    cu_k: np.ndarray


def seeded_lengths(seed: int, n: int, lo: int, hi: int, stream: int = 0) -> tuple:
    """``n`` lengths uniform in [lo, hi] from the counter-based generator."""
    key = stream_key(seed, TID_LENGTHS)
    return tuple(lo + (u64_int(key, (stream << 32) + i) * (hi - lo + 1) >> 64) for i in range(n))


def generate_varlen(wl: VarlenWorkload) -> VarlenInputs:
    """Draw packed Q, K, V for ``wl``: element (t, h, c) of the packed tensor is
    element (0, t, h, c) of a B=1 BSHD draw of the same generator."""
    if len(wl.lengths_k) != len(wl.lengths_q) or wl.H % wl.H_kv:
        raise ValueError("lengths_q and lengths_k differ in count, or H is not a multiple of H_kv")
    cu_q = np.concatenate([[0], np.cumsum(wl.lengths_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(wl.lengths_k)]).astype(np.int32)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = normal_bf16(wl.seed, TID_Q, max(tq, 1) * wl.H * D).reshape(-1, wl.H, D)[:tq]
    k = normal_bf16(wl.seed, TID_K, max(tk, 1) * wl.H_kv * D).reshape(-1, wl.H_kv, D)[:tk]
    v = normal_bf16(wl.seed, TID_V, max(tk, 1) * wl.H_kv * D).reshape(-1, wl.H_kv, D)[:tk]
    return VarlenInputs(wl, np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v), cu_q, cu_k)


VARLEN_WORKLOADS = {
    # 16 causal sequences of 256 .. 8192 tokens (about 66K in all), 32 query heads over 8 K/V heads
    "varlen_mix": VarlenWorkload("varlen_mix", seeded_lengths(0, 16, 256, 8192), seeded_lengths(0, 16, 256, 8192),
                                 32, 8, ("rtne",), mask="causal"),
}
