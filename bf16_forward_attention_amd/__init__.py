"""Fused bf16 forward attention (head_dim 128) for MI355X: without a mask or with a
causal one, grouped K/V heads, packed variable-length batches, per-row log-sum-exp.

Thin binding over the C ABI in ``include/attn_fwd.h``: argument marshalling
only, every step of the computation runs in the HIP library
``libattn_fwd.so``.  PyTorch is used for device memory and streams.

    attn_fwd_bf16(q, k, v, o, B, H, Sq, Sk, layout, round_mode, stream) -> status
    attn_fwd_bf16_masked(q, k, v, o, B, H, Sq, Sk, layout, round_mode, mask, stream) -> status
    attn_fwd_bf16_gqa(q, k, v, o, lse, B, H, H_kv, Sq, Sk, layout, round_mode, mask, stream) -> status
    attn_fwd_bf16_varlen(q, k, v, o, lse, cu_q, cu_k, B, H, H_kv, total_q, total_k, max_seqlen_q, round_mode,
                         mask, stream) -> status
    attn_fwd_bf16_ws(q, k, v, o, B, H, Sq, Sk, layout, round_mode, ws, ws_bytes, stream) -> status
    attn_fwd_bf16_workspace_size(B, H, Sq, Sk) -> bytes
    attn_fwd_bf16_gqa_ws(q, k, v, o, lse, B, H, H_kv, Sq, Sk, layout, round_mode, mask, ws, ws_bytes,
                         stream) -> status
    attn_fwd_bf16_gqa_workspace_size(B, H, Sq, Sk, mask) -> bytes
    attn_fwd_bf16_gqa_noalloc(q, k, v, o, lse, B, H, H_kv, Sq, Sk, layout, round_mode, mask, stream) -> status
    attn_fwd_bf16_partial(q, k, v, o_part, lse_part, B, H, H_kv, Sq, Sk, key_offset, Sk_total, layout, mask,
                          stream) -> status
    attn_fwd_bf16_merge(o_parts, lse_parts, n_parts, o, lse, B, H, Sq, layout, round_mode, stream) -> status
    attn_fwd_bf16_split_plan(n_work, n_tiles, n_cu) -> (whole, split items, splits, tiles per split)
    attn_fwd_bf16_split_plan_masked(n_heads, Sq, Sk, mask, n_cu) -> the same four numbers
    attn_fwd(q, k, v, out=None, layout="bshd", round_mode="rtne", split=True, mask="none") -> torch.Tensor
    attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, out=None, round_mode="rtne",
                    mask="none") -> torch.Tensor
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "attn_fwd_bf16", "attn_fwd_bf16_masked", "attn_fwd_bf16_gqa", "attn_fwd_bf16_varlen", "attn_fwd_bf16_ws",
    "attn_fwd_varlen", "attn_fwd_bf16_workspace_size", "attn_fwd_bf16_gqa_ws", "attn_fwd_bf16_gqa_workspace_size",
    "attn_fwd_bf16_split_plan", "attn_fwd_bf16_split_plan_masked", "attn_fwd_bf16_partial", "attn_fwd_bf16_merge", "attn_fwd_bf16_strerror", "attn_fwd_bf16_abi_version", "attn_fwd",
    "AttnError", "LAYOUTS", "ROUND_MODES", "MASKS", "library_path", "load_library",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libattn_fwd.so")

# values of attn_layout_t / attn_round_t in include/attn_fwd.h
LAYOUTS = {"bshd": 0, "bhsd": 1}
ROUND_MODES = {"rtne": 0, "rtna": 1, "rtz": 2}
# values of attn_mask_t: query row i attends to keys j <= i + off, off = 0 or Sk - Sq
MASKS = {"none": 0, "causal": 1, "causal_br": 2}
HEAD_DIM = 128

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"attn_fwd_bf16 failed ({status}): {attn_fwd_bf16_strerror(status)}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load the built HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                f"{_LIB_PATH} is missing: build it with `python -m bf16_forward_attention_amd.build` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.attn_fwd_bf16.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, vp]
        lib.attn_fwd_bf16.restype = ctypes.c_int
        lib.attn_fwd_bf16_masked.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, vp]
        lib.attn_fwd_bf16_masked.restype = ctypes.c_int
        lib.attn_fwd_bf16_gqa.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, vp]
        lib.attn_fwd_bf16_gqa.restype = ctypes.c_int
        lib.attn_fwd_bf16_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                             ctypes.c_int, vp]
        lib.attn_fwd_bf16_varlen.restype = ctypes.c_int
        lib.attn_fwd_bf16_ws.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, vp, i64,
                                         vp]
        lib.attn_fwd_bf16_ws.restype = ctypes.c_int
        lib.attn_fwd_bf16_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64)]
        lib.attn_fwd_bf16_workspace_size.restype = ctypes.c_int
        lib.attn_fwd_bf16_split_plan.argtypes = [i64, i64, i64, ctypes.POINTER(i64)]
        lib.attn_fwd_bf16_split_plan.restype = ctypes.c_int
        lib.attn_fwd_bf16_gqa_ws.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, vp, i64, vp]
        lib.attn_fwd_bf16_gqa_ws.restype = ctypes.c_int
        lib.attn_fwd_bf16_gqa_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int,
                                                  ctypes.c_int, ctypes.c_int, vp]
        lib.attn_fwd_bf16_gqa_noalloc.restype = ctypes.c_int
        lib.attn_fwd_bf16_gqa_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.POINTER(i64)]
        lib.attn_fwd_bf16_gqa_workspace_size.restype = ctypes.c_int
        lib.attn_fwd_bf16_split_plan_masked.argtypes = [i64, i64, i64, ctypes.c_int, i64, ctypes.POINTER(i64)]
        lib.attn_fwd_bf16_split_plan_masked.restype = ctypes.c_int
        lib.attn_fwd_bf16_partial.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                              ctypes.c_int, vp]
        lib.attn_fwd_bf16_partial.restype = ctypes.c_int
        lib.attn_fwd_bf16_merge.argtypes = [vp, vp, i64, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, vp]
        lib.attn_fwd_bf16_merge.restype = ctypes.c_int
        lib.attn_fwd_bf16_strerror.argtypes = [ctypes.c_int]
        lib.attn_fwd_bf16_strerror.restype = ctypes.c_char_p
        lib.attn_fwd_bf16_abi_version.argtypes = []
        lib.attn_fwd_bf16_abi_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def attn_fwd_bf16(q: int, k: int, v: int, o: int, B: int, H: int, Sq: int, Sk: int,
                  layout: int, round_mode: int, stream: int) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return load_library().attn_fwd_bf16(q, k, v, o, B, H, Sq, Sk, layout, round_mode, stream)


def attn_fwd_bf16_masked(q: int, k: int, v: int, o: int, B: int, H: int, Sq: int, Sk: int,
                         layout: int, round_mode: int, mask: int, stream: int) -> int:
    """The masked C entry point with raw device addresses; returns the status code."""
    return load_library().attn_fwd_bf16_masked(q, k, v, o, B, H, Sq, Sk, layout, round_mode, mask, stream)


def attn_fwd_bf16_gqa(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, H_kv: int, Sq: int, Sk: int,
                      layout: int, round_mode: int, mask: int, stream: int) -> int:
    """The grouped-query C entry point with raw device addresses (lse 0: not
    written); returns the status code."""
    return load_library().attn_fwd_bf16_gqa(q, k, v, o, lse or None, B, H, H_kv, Sq, Sk, layout, round_mode, mask,
                                            stream)


def attn_fwd_bf16_varlen(q: int, k: int, v: int, o: int, lse: int, cu_q: int, cu_k: int, B: int, H: int,
                         H_kv: int, total_q: int, total_k: int, max_seqlen_q: int, round_mode: int, mask: int,
                         stream: int) -> int:
    """The variable-length C entry point with raw device addresses (lse 0: not
    written); returns the status code."""
    return load_library().attn_fwd_bf16_varlen(q, k, v, o, lse or None, cu_q, cu_k, B, H, H_kv, total_q, total_k,
                                               max_seqlen_q, round_mode, mask, stream)


def attn_fwd_bf16_ws(q: int, k: int, v: int, o: int, B: int, H: int, Sq: int, Sk: int, layout: int,
                     round_mode: int, workspace: int, workspace_bytes: int, stream: int) -> int:
    """The key-range-splitting C entry point; returns the status code."""
    return load_library().attn_fwd_bf16_ws(q, k, v, o, B, H, Sq, Sk, layout, round_mode, workspace,
                                           workspace_bytes, stream)


def attn_fwd_bf16_workspace_size(B: int, H: int, Sq: int, Sk: int) -> int:
    """Workspace bytes attn_fwd_bf16_ws needs on the current device (raises AttnError)."""
    out = ctypes.c_int64(0)
    status = load_library().attn_fwd_bf16_workspace_size(B, H, Sq, Sk, ctypes.byref(out))
    if status != 0:
        raise AttnError(status)
    return out.value


def attn_fwd_bf16_gqa_ws(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, H_kv: int, Sq: int, Sk: int,
                         layout: int, round_mode: int, mask: int, workspace: int, workspace_bytes: int,
                         stream: int) -> int:
    """The grouped-query, masked C entry point allowed to split the key range
    (lse 0: not written); returns the status code."""
    return load_library().attn_fwd_bf16_gqa_ws(q, k, v, o, lse or None, B, H, H_kv, Sq, Sk, layout, round_mode,
                                               mask, workspace or None, workspace_bytes, stream)


def attn_fwd_bf16_gqa_noalloc(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, H_kv: int, Sq: int,
                              Sk: int, layout: int, round_mode: int, mask: int, stream: int) -> int:
    """attn_fwd_bf16_gqa_ws with the library's static scratch instead of a workspace
    (allocates nothing; lse 0: not written); returns the status code."""
    return load_library().attn_fwd_bf16_gqa_noalloc(q, k, v, o, lse or None, B, H, H_kv, Sq, Sk, layout,
                                                    round_mode, mask, stream)


def attn_fwd_bf16_gqa_workspace_size(B: int, H: int, Sq: int, Sk: int, mask: int) -> int:
    """Workspace bytes attn_fwd_bf16_gqa_ws needs on the current device (raises AttnError)."""
    out = ctypes.c_int64(0)
    status = load_library().attn_fwd_bf16_gqa_workspace_size(B, H, Sq, Sk, mask, ctypes.byref(out))
    if status != 0:
        raise AttnError(status)
    return out.value


def attn_fwd_bf16_split_plan_masked(n_heads: int, Sq: int, Sk: int, mask: int, n_cu: int):
    """attn_fwd_bf16_gqa_ws's split decision: (items run whole, items split,
    ranges per split item, tiles per range of the heaviest item)."""
    out = (ctypes.c_int64 * 4)()
    status = load_library().attn_fwd_bf16_split_plan_masked(n_heads, Sq, Sk, mask, n_cu, out)
    if status != 0:
        raise AttnError(status)
    return tuple(out)


def attn_fwd_bf16_partial(q: int, k: int, v: int, o_part: int, lse_part: int, B: int, H: int, H_kv: int, Sq: int,
                          Sk: int, key_offset: int, Sk_total: int, layout: int, mask: int, stream: int) -> int:
    """One key shard's fp32 rows and log-sum-exp (raw device addresses); returns the status code."""
    return load_library().attn_fwd_bf16_partial(q, k, v, o_part or None, lse_part or None, B, H, H_kv, Sq, Sk,
                                                key_offset, Sk_total, layout, mask, stream)


def attn_fwd_bf16_merge(o_parts: int, lse_parts: int, n_parts: int, o: int, lse: int, B: int, H: int, Sq: int,
                        layout: int, round_mode: int, stream: int) -> int:
    """Merge of key-shard partials into the bf16 output (lse 0: not written); returns the status code."""
    return load_library().attn_fwd_bf16_merge(o_parts or None, lse_parts or None, n_parts, o or None, lse or None,
                                              B, H, Sq, layout, round_mode, stream)


def attn_fwd_bf16_split_plan(n_work: int, n_tiles: int, n_cu: int):
    """(items run whole, items split, ranges per split item, tiles per range)."""
    out = (ctypes.c_int64 * 4)()
    status = load_library().attn_fwd_bf16_split_plan(n_work, n_tiles, n_cu, out)
    if status != 0:
        raise AttnError(status)
    return tuple(out)


def attn_fwd_bf16_strerror(status: int) -> str:
    return load_library().attn_fwd_bf16_strerror(status).decode()


def attn_fwd_bf16_abi_version() -> int:
    return load_library().attn_fwd_bf16_abi_version()


def _dims(q, k, layout: str):
    if layout == "bshd":
        B, Sq, H, d = q.shape
        Bk, Sk, Hk, dk = k.shape
    elif layout == "bhsd":
        B, H, Sq, d = q.shape
        Bk, Hk, Sk, dk = k.shape
    else:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}, got {layout!r}")
    if d != HEAD_DIM or dk != HEAD_DIM or Bk != B or Hk < 1 or H % Hk:
        raise ValueError(f"incompatible shapes q{tuple(q.shape)} k{tuple(k.shape)} for layout {layout}")
    return B, H, Hk, Sq, Sk


def _record_on(s, stream, *tensors):
    """Tensors allocated here on torch's current stream but written on a caller's other stream:
    tell torch's caching allocator, so that their memory is not handed out again before that
    stream is done with it."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(s)


def attn_fwd(q, k, v, out=None, layout: str = "bshd", round_mode: str = "rtne", stream=None,
             split: bool = True, mask: str = "none", with_lse: bool = False):
    """O = softmax(Q K^T / sqrt(128)) V on bf16 CUDA(HIP) tensors.

    ``q`` [B,Sq,H,128] and ``k``/``v`` [B,Sk,H_kv,128] for "bshd", or
    [B,H,S,128] / [B,H_kv,S,128] for "bhsd"; all contiguous bf16 on one
    device.  H_kv < H (a divisor of H) is grouped-query attention through
    attn_fwd_bf16_gqa.  Enqueued on
    ``stream`` (default: torch's current stream on that device).  With
    ``split`` the key range may be split (attn_fwd_bf16_ws, workspace from
    torch; attn_fwd_bf16_gqa_ws with a mask, grouped heads or lse); without,
    the single-pass entry points.  ``mask`` "causal" or "causal_br" lets row
    i see keys j <= i or j <= i + Sk - Sq only.  ``with_lse`` returns
    ``(out, lse)`` with lse [B, H, Sq] fp32, each row's log-sum-exp.
    """
    import torch

    if round_mode not in ROUND_MODES:
        raise ValueError(f"round_mode must be one of {sorted(ROUND_MODES)}, got {round_mode!r}")
    if mask not in MASKS:
        raise ValueError(f"mask must be one of {sorted(MASKS)}, got {mask!r}")
    B, H, H_kv, Sq, Sk = _dims(q, k, layout)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("v must have the shape of k")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 GPU tensor")
        if t.device != q.device:
            raise ValueError("q, k and v must be on one device")
    own_out = out is None
    if own_out:
        out = torch.empty_like(q)
    elif (out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(q.shape) or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q on q's device")
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device) if with_lse else None
        direct = mask == "none" and H_kv == H and not with_lse
        ws_bytes = 0
        if split:
            ws_bytes = (attn_fwd_bf16_workspace_size(B, H, Sq, Sk) if direct
                        else attn_fwd_bf16_gqa_workspace_size(B, H, Sq, Sk, MASKS[mask]))
        if ws_bytes > 0 and not direct:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
            status = attn_fwd_bf16_gqa_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                          lse.data_ptr() if with_lse else 0, B, H, H_kv, Sq, Sk, LAYOUTS[layout],
                                          ROUND_MODES[round_mode], MASKS[mask], ws.data_ptr(), ws_bytes,
                                          s.cuda_stream)
            ws.record_stream(s)
        elif H_kv != H or with_lse:
            status = attn_fwd_bf16_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       lse.data_ptr() if with_lse else 0, B, H, H_kv, Sq, Sk, LAYOUTS[layout],
                                       ROUND_MODES[round_mode], MASKS[mask], s.cuda_stream)
        elif mask != "none":
            status = attn_fwd_bf16_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, Sq, Sk,
                                          LAYOUTS[layout], ROUND_MODES[round_mode], MASKS[mask], s.cuda_stream)
        elif ws_bytes > 0:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
            status = attn_fwd_bf16_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, Sq, Sk,
                                      LAYOUTS[layout], ROUND_MODES[round_mode], ws.data_ptr(), ws_bytes,
                                      s.cuda_stream)
            ws.record_stream(s)
        else:
            status = attn_fwd_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, Sq, Sk,
                                   LAYOUTS[layout], ROUND_MODES[round_mode], s.cuda_stream)
        _record_on(s, stream, out if own_out else None, lse)
    if status != 0:
        raise AttnError(status)
    return (out, lse) if with_lse else out


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, out=None, round_mode: str = "rtne",
                    mask: str = "none", stream=None, with_lse: bool = False):
    """Variable-length batch: ``q`` [total_q, H, 128], ``k``/``v`` [total_k, H_kv, 128]
    bf16 and ``cu_seqlens_q``/``cu_seqlens_k`` int32 [B+1] offsets, all on one
    device; sequence b attends within its own rows (attn_fwd_bf16_varlen).
    ``max_seqlen_q`` must be at least every sequence's query length.
    ``with_lse`` returns ``(out, lse)`` with lse [H, total_q] fp32."""
    import torch

    if round_mode not in ROUND_MODES or mask not in MASKS:
        raise ValueError(f"round_mode must be one of {sorted(ROUND_MODES)} and mask one of {sorted(MASKS)}")
    if q.dim() != 3 or k.dim() != 3 or q.shape[2] != HEAD_DIM or k.shape[2] != HEAD_DIM or v.shape != k.shape:
        raise ValueError(f"expected q [total_q, H, 128] and k, v [total_k, H_kv, 128], got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous bfloat16 GPU tensor on q's device")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous int32 vector on q's device")
    if cu_seqlens_k.numel() != cu_seqlens_q.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B+1 >= 2 offsets")
    total_q, H, _ = q.shape
    total_k, H_kv, _ = k.shape
    own_out = out is None
    if own_out:
        out = torch.empty_like(q)
    elif (out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(q.shape) or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q on q's device")
    lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device) if with_lse else None
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        status = attn_fwd_bf16_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      lse.data_ptr() if with_lse else 0,
                                      cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), cu_seqlens_q.numel() - 1,
                                      H, H_kv, total_q, total_k, max_seqlen_q, ROUND_MODES[round_mode], MASKS[mask],
                                      s.cuda_stream)
        _record_on(s, stream, out if own_out else None, lse)
    if status != 0:
        raise AttnError(status)
    return (out, lse) if with_lse else out
