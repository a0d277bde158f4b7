"""Plain fp64 CPU oracle for bf16 forward attention (d = 128), unmasked or causal,
with as many K/V heads as query heads or fewer (grouped-query attention).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product path never does.
It shares no code with the HIP library (see ``attn_oracle.c`` for what is
computed and the passages it follows).

Parity status of each function (what pins it, in ``tests/test_oracle_*.py``):

* ``decode_bf16``   -- exhaustive over all 65,536 patterns vs the float32
                       bit-extension identity.
* ``round_bf16``    -- closed forms over structured float32 patterns, a
                       library RNE cross-check (torch CPU), and a
                       definitional nearest-neighbour search with exact
                       rationals on random and tie binary64 inputs.
* ``attn_rows``     -- closed forms (uniform logits, dominant logit, Sk = 1,
                       two-key logistic), midpoint ties, invariants, NaN/Inf
                       rules, mpmath brute force on tiny inputs and a torch
                       float64 softmax cross-check.  With a causal ``mask``:
                       the first row of a top-left diagonal returns V_0, a row
                       equals the unmasked oracle on its visible keys, keys
                       past the diagonal cannot change it, rows with no
                       visible key are NaN, mpmath brute force, and torch's
                       float64 attention with its top-left (``is_causal``) and
                       bottom-right (``causal_lower_right``) masks.  With
                       fewer K/V heads (read from k's shape): equal, bit for
                       bit, to the one-head-per-query-head oracle on K/V
                       heads repeated group-wise, and torch's float64
                       attention with ``enable_gqa``.
* ``attn_rows_varlen`` -- sequences packed one after another: each is the
                       fixed-length attention above on its own rows.  Pinned
                       by torch's float64 attention run per sequence, a
                       dominant key per sequence (catches rows or keys taken
                       from a neighbour), and mutants of the slicing.
* ``softmax_row``   -- rows sum to one; agrees with a library softmax.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

MODES = {"rtne": 0, "rtna": 1, "rtz": 2}
LAYOUTS = {"bshd": 0, "bhsd": 1}
# query row i attends to keys j <= i + off: off = 0 ("causal", top left) or Sk - Sq ("causal_br")
MASKS = {"none": 0, "causal": 1, "causal_br": 2}
D = 128

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
               "-pthread", _SRC, "-lm", "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # ORACLE_LIB lets the mutation tests load a deliberately broken build
        path = os.environ.get("ORACLE_LIB")
        if not path:
            if not os.path.exists(_LIB):
                build()
            path = _LIB
        lib = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_decode.restype = ctypes.c_double
        lib.oracle_round_bf16.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_round_array.argtypes = [f64p, i64, ctypes.c_int, u16p]
        lib.oracle_round_array.restype = None
        lib.oracle_decode_array.argtypes = [u16p, i64, f64p]
        lib.oracle_decode_array.restype = None
        lib.oracle_attn_rows.argtypes = [u16p, u16p, u16p, i64, i64, i64, i64, ctypes.c_int,
                                         i64p, i64, f64p, u16p, ctypes.c_int]
        lib.oracle_attn_rows.restype = ctypes.c_int
        lib.oracle_attn_rows_masked.argtypes = [u16p, u16p, u16p, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                                i64p, i64, f64p, u16p, ctypes.c_int]
        lib.oracle_attn_rows_masked.restype = ctypes.c_int
        lib.oracle_attn_rows_gqa.argtypes = [u16p, u16p, u16p, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                             i64p, i64, f64p, u16p, f64p, ctypes.c_int]
        lib.oracle_attn_rows_gqa.restype = ctypes.c_int
        lib.oracle_softmax_row.argtypes = [u16p, u16p, i64, i64, i64, i64, ctypes.c_int,
                                           i64, i64, i64, f64p]
        lib.oracle_softmax_row.restype = ctypes.c_double
        _lib = lib
    return _lib


def _u16(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _f64(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """Exact binary64 values of bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_decode_array(_u16(b), b.size, _f64(out))
    return out


def round_bf16(x: np.ndarray, mode: str) -> np.ndarray:
    """bf16 bits of binary64 values rounded once in ``mode``."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_round_array(_f64(a), a.size, MODES[mode], _u16(out))
    return out


def _check_inputs(q, k, v, B, H, H_kv, Sq, Sk, layout):
    if H_kv < 1 or H % H_kv:
        raise ValueError(f"the {H} query heads are not a multiple of the {H_kv} K/V heads")
    shape_q = (B, Sq, H, D) if layout == "bshd" else (B, H, Sq, D)
    shape_k = (B, Sk, H_kv, D) if layout == "bshd" else (B, H_kv, Sk, D)
    for name, t, shp in (("q", q, shape_q), ("k", k, shape_k), ("v", v, shape_k)):
        if t.dtype != np.uint16 or tuple(t.shape) != shp or not t.flags.c_contiguous:
            raise ValueError(f"{name}: expected contiguous uint16 {shp}, got {t.dtype} {t.shape}")


def attn_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, layout: str, rows, nthreads: int | None = None,
              mask: str = "none", with_lse: bool = False):
    """Exact outputs of the given (b, h, i) query rows and their roundings.

    ``q``/``k``/``v`` are bf16 bit arrays stored in ``layout`` (k and v may
    hold fewer heads than q: grouped-query attention); ``mask`` is one of
    ``MASKS``.  Returns
    ``(o_exact, o_round)``: ``o_exact`` is float64 [n, 128] and ``o_round``
    uint16 [n, 3, 128] in the mode order RTNE, RTNA, RTZ; both follow the
    order of ``rows``.  With ``with_lse`` a third array holds each row's
    log-sum-exp (float64 [n]; see attn_oracle.c for its special values).
    """
    if layout == "bshd":
        B, Sq, H, _ = q.shape
        Sk, H_kv = k.shape[1], k.shape[2]
    else:
        B, H, Sq, _ = q.shape
        H_kv, Sk = k.shape[1], k.shape[2]
    _check_inputs(q, k, v, B, H, H_kv, Sq, Sk, layout)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    n = rows.shape[0]
    order = np.lexsort((rows[:, 2], rows[:, 1], rows[:, 0]))
    srt = np.ascontiguousarray(rows[order])
    o_exact = np.empty((n, D), dtype=np.float64)
    o_round = np.empty((n, 3, D), dtype=np.uint16)
    lse = np.empty(n, dtype=np.float64)
    if mask not in MASKS:
        raise ValueError(f"mask must be one of {sorted(MASKS)}, got {mask!r}")
    rc = _load().oracle_attn_rows_gqa(_u16(q), _u16(k), _u16(v), B, H, H_kv, Sq, Sk, LAYOUTS[layout], MASKS[mask],
                                      srt.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n,
                                      _f64(o_exact), _u16(o_round), _f64(lse), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_attn_rows failed with {rc}")
    inv = np.empty_like(order)
    inv[order] = np.arange(n)
    if with_lse:
        return o_exact[inv], o_round[inv], lse[inv]
    return o_exact[inv], o_round[inv]


def attn_all(q, k, v, layout: str, nthreads: int | None = None, mask: str = "none"):
    """Every row: o_exact [B,H,Sq,128] and o_round [3,B,H,Sq,128] (logical order)."""
    if layout == "bshd":
        B, Sq, H, _ = q.shape
    else:
        B, H, Sq, _ = q.shape
    bb, hh, ii = np.meshgrid(np.arange(B), np.arange(H), np.arange(Sq), indexing="ij")
    rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    ex, rd = attn_rows(q, k, v, layout, rows, nthreads, mask)
    return ex.reshape(B, H, Sq, D), np.moveaxis(rd.reshape(B, H, Sq, 3, D), 3, 0)


def softmax_row(q, k, layout: str, b: int, h: int, i: int):
    """Normalised softmax weights w_j / l of one row, and l."""
    if layout == "bshd":
        B, Sq, H, _ = q.shape
        Sk = k.shape[1]
    else:
        B, H, Sq, _ = q.shape
        Sk = k.shape[2]
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    w = np.empty(Sk, dtype=np.float64)
    l = _load().oracle_softmax_row(_u16(q), _u16(k), B, H, Sq, Sk, LAYOUTS[layout], b, h, i, _f64(w))
    return w, l


def attn_rows_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k, rows, mask: str = "none",
                     nthreads: int | None = None, with_lse: bool = False):
    """Exact outputs of packed query rows of a variable-length batch.

    ``q`` is [total_q, H, 128] and ``k``/``v`` [total_k, H_kv, 128] bf16 bits:
    sequence b holds query rows cu_q[b] .. cu_q[b+1]-1 and key rows
    cu_k[b] .. cu_k[b+1]-1, and attends only within itself (variable-length
    batching in FlashAttention's packed "cu_seqlens" layout).
    Each sequence is the fixed-length problem B=1, Sq = its query rows, Sk = its
    key rows in BSHD, handed to ``attn_rows`` as such; a sequence with no key
    gives NaN rows (the 0/0 of an empty softmax).  ``rows`` are (t, h) pairs
    of packed query row and head.  Returns ``(o_exact, o_round)`` like
    ``attn_rows`` (and the log-sum-exp of each row with ``with_lse``: -Inf for
    a sequence without keys).
    """
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    B = len(cu_q) - 1
    if len(cu_k) != B + 1 or cu_q[0] != 0 or cu_k[0] != 0 or np.any(np.diff(cu_q) < 0) or np.any(np.diff(cu_k) < 0):
        raise ValueError("cu_q / cu_k must be non-decreasing offsets starting at 0, one more than the sequences")
    if cu_q[-1] != q.shape[0] or cu_k[-1] != k.shape[0] or v.shape != k.shape:
        raise ValueError("the offsets do not cover the packed tensors")
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    n = rows.shape[0]
    o_exact = np.full((n, D), np.nan)
    o_round = np.full((n, 3, D), 0x7FC0, dtype=np.uint16)
    lse = np.full(n, -np.inf)
    seq = np.searchsorted(cu_q, rows[:, 0], side="right") - 1
    for b in np.unique(seq):
        sel = np.nonzero(seq == b)[0]
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if k1 == k0:
            continue  # no key: NaN rows
        sub = [(0, int(h), int(t - q0)) for t, h in rows[sel]]
        ex, rd, ls = attn_rows(np.ascontiguousarray(q[q0:q1][None]), np.ascontiguousarray(k[k0:k1][None]),
                               np.ascontiguousarray(v[k0:k1][None]), "bshd", sub, nthreads, mask, with_lse=True)
        o_exact[sel] = ex
        o_round[sel] = rd
        lse[sel] = ls
    if with_lse:
        return o_exact, o_round, lse
    return o_exact, o_round


def attn_all_varlen(q, k, v, cu_q, cu_k, mask: str = "none", nthreads: int | None = None):
    """Every packed row: o_exact [total_q, H, 128] and o_round [3, total_q, H, 128]."""
    total_q, H, _ = q.shape
    tt, hh = np.meshgrid(np.arange(total_q), np.arange(H), indexing="ij")
    rows = np.stack([tt.ravel(), hh.ravel()], axis=1)
    ex, rd = attn_rows_varlen(q, k, v, cu_q, cu_k, rows, mask, nthreads)
    return ex.reshape(total_q, H, D), np.moveaxis(rd.reshape(total_q, H, 3, D), 2, 0)
