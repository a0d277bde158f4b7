"""Helpers for the GPU tests: move bf16 bit arrays to the device, call the
library through its C ABI, bring the output back as bits."""
from __future__ import annotations

import sys

import numpy as np
import torch

import bf16_forward_attention_amd as attn
from bf16_forward_attention_amd import synth

MODES = ("rtne", "rtna", "rtz")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_device(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda:0")


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def launch(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, layout: str, mode: str,
           stream: torch.cuda.Stream | None = None) -> None:
    """Call attn_fwd_bf16 through the C ABI with raw device pointers."""
    if layout == "bshd":
        B, Sq, H, _ = q.shape
        Sk = k.shape[1]
    else:
        B, H, Sq, _ = q.shape
        Sk = k.shape[2]
    s = stream if stream is not None else torch.cuda.current_stream()
    st = attn.attn_fwd_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, Sq, Sk,
                            attn.LAYOUTS[layout], attn.ROUND_MODES[mode], s.cuda_stream)
    if st != 0:
        raise attn.AttnError(st)


def launch_masked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, layout: str, mode: str,
                  mask: str, stream: torch.cuda.Stream | None = None) -> None:
    """Call attn_fwd_bf16_masked through the C ABI with raw device pointers."""
    if layout == "bshd":
        B, Sq, H, _ = q.shape
        Sk = k.shape[1]
    else:
        B, H, Sq, _ = q.shape
        Sk = k.shape[2]
    s = stream if stream is not None else torch.cuda.current_stream()
    st = attn.attn_fwd_bf16_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, Sq, Sk,
                                   attn.LAYOUTS[layout], attn.ROUND_MODES[mode], attn.MASKS[mask], s.cuda_stream)
    if st != 0:
        raise attn.AttnError(st)


def launch_gqa(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, layout: str, mode: str,
               mask: str = "none", stream: torch.cuda.Stream | None = None, lse: torch.Tensor | None = None) -> None:
    """Call attn_fwd_bf16_gqa through the C ABI; the K/V head count comes from k's shape."""
    if layout == "bshd":
        B, Sq, H, _ = q.shape
        Sk, H_kv = k.shape[1], k.shape[2]
    else:
        B, H, Sq, _ = q.shape
        H_kv, Sk = k.shape[1], k.shape[2]
    s = stream if stream is not None else torch.cuda.current_stream()
    st = attn.attn_fwd_bf16_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr() if lse is not None else 0, B, H, H_kv, Sq, Sk,
                                attn.LAYOUTS[layout], attn.ROUND_MODES[mode], attn.MASKS[mask], s.cuda_stream)
    if st != 0:
        raise attn.AttnError(st)


def launch_ws(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, layout: str, mode: str,
              stream: torch.cuda.Stream | None = None) -> int:
    """Call attn_fwd_bf16_ws (key ranges split when it pays) with a torch-allocated
    workspace of the size the library asks for; returns that size."""
    if layout == "bshd":
        B, Sq, H, _ = q.shape
        Sk = k.shape[1]
    else:
        B, H, Sq, _ = q.shape
        Sk = k.shape[2]
    s = stream if stream is not None else torch.cuda.current_stream()
    nbytes = attn.attn_fwd_bf16_workspace_size(B, H, Sq, Sk)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    st = attn.attn_fwd_bf16_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, Sq, Sk,
                               attn.LAYOUTS[layout], attn.ROUND_MODES[mode], ws.data_ptr(), nbytes, s.cuda_stream)
    if st != 0:
        raise attn.AttnError(st)
    torch.cuda.synchronize()
    return nbytes


def launch_gqa_ws(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, layout: str, mode: str,
                  mask: str = "none", lse: torch.Tensor | None = None) -> int:
    """Call attn_fwd_bf16_gqa_ws through the C ABI with a torch-allocated
    workspace of the size the library asks for; returns that size."""
    if layout == "bshd":
        B, Sq, H, _ = q.shape
        Sk, H_kv = k.shape[1], k.shape[2]
    else:
        B, H, Sq, _ = q.shape
        H_kv, Sk = k.shape[1], k.shape[2]
    s = torch.cuda.current_stream()
    nbytes = attn.attn_fwd_bf16_gqa_workspace_size(B, H, Sq, Sk, attn.MASKS[mask])
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    st = attn.attn_fwd_bf16_gqa_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr() if lse is not None else 0, B, H, H_kv, Sq, Sk,
                                   attn.LAYOUTS[layout], attn.ROUND_MODES[mode], attn.MASKS[mask], ws.data_ptr(),
                                   nbytes, s.cuda_stream)
    if st != 0:
        raise attn.AttnError(st)
    torch.cuda.synchronize()
    return nbytes


class Dev:
    """Device copies of one Inputs bundle."""

    def __init__(self, inp: synth.Inputs):
        self.inp = inp
        self.layout = inp.wl.layout
        self.q, self.k, self.v = to_device(inp.q), to_device(inp.k), to_device(inp.v)
        self.o = torch.empty_like(self.q)

    def run(self, mode: str, split: bool = False, mask: str | None = None) -> np.ndarray:
        """Output bits in the stored layout (split: through attn_fwd_bf16_ws, or
        attn_fwd_bf16_gqa_ws with a mask or grouped heads; otherwise a mask, or
        the workload's own, through attn_fwd_bf16_masked, grouped heads through
        attn_fwd_bf16_gqa)."""
        mask = self.inp.wl.mask if mask is None else mask
        grouped = self.inp.wl.kv_heads != self.inp.wl.H
        if split and (grouped or mask != "none"):
            launch_gqa_ws(self.q, self.k, self.v, self.o, self.layout, mode, mask)
        elif grouped:
            launch_gqa(self.q, self.k, self.v, self.o, self.layout, mode, mask)
        elif mask != "none":
            launch_masked(self.q, self.k, self.v, self.o, self.layout, mode, mask)
        elif split:
            launch_ws(self.q, self.k, self.v, self.o, self.layout, mode)
        else:
            launch(self.q, self.k, self.v, self.o, self.layout, mode)
        torch.cuda.synchronize()
        return to_bits(self.o)

    def run_logical(self, mode: str, split: bool = False, mask: str | None = None) -> np.ndarray:
        return np.ascontiguousarray(synth.to_logical(self.run(mode, split, mask), self.layout))


def run_raw(q, k, v, layout: str, mode: str, mask: str = "none") -> np.ndarray:
    """Stored-layout bits in, stored-layout bits out."""
    dq, dk, dv = to_device(q), to_device(k), to_device(v)
    o = torch.empty_like(dq)
    if mask == "none":
        launch(dq, dk, dv, o, layout, mode)
    else:
        launch_masked(dq, dk, dv, o, layout, mode, mask)
    torch.cuda.synchronize()
    return to_bits(o)


def run_logical(q, k, v, layout: str, mode: str, mask: str = "none") -> np.ndarray:
    """Logical [B,H,S,128] bits in and out, stored in ``layout`` on the way."""
    out = run_raw(synth.to_layout(q, layout), synth.to_layout(k, layout), synth.to_layout(v, layout), layout, mode,
                  mask)
    return np.ascontiguousarray(synth.to_logical(out, layout))
