"""The C ABI: the built library exports what include/attn_fwd.h declares, the
enum values agree with the Python binding, and argument errors come back
before any HIP call (so these run without a GPU)."""
import os
import re
import subprocess

import pytest

import bf16_forward_attention_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_fwd.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_fwd_\w+)\s*\(", text, re.M)))


def _enum_values():
    text = open(HEADER).read()
    return {name: int(val) for name, val in re.findall(r"\b(ATTN_\w+)\s*=\s*(\d+)", text)}


def test_library_exports_every_declared_symbol():
    funcs = _declared_functions()
    assert funcs == ["attn_fwd_bf16", "attn_fwd_bf16_abi_version", "attn_fwd_bf16_gqa", "attn_fwd_bf16_gqa_noalloc",
                     "attn_fwd_bf16_gqa_workspace_size", "attn_fwd_bf16_gqa_ws", "attn_fwd_bf16_masked", "attn_fwd_bf16_merge", "attn_fwd_bf16_partial",
                     "attn_fwd_bf16_split_plan", "attn_fwd_bf16_split_plan_masked", "attn_fwd_bf16_strerror",
                     "attn_fwd_bf16_varlen",
                     "attn_fwd_bf16_workspace_size", "attn_fwd_bf16_ws"]
    out = subprocess.run(["nm", "-D", "--defined-only", attn.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, re.M))
    for f in funcs:
        assert f in exported, f
    lib = attn.load_library()
    for f in funcs:
        assert hasattr(lib, f)


def test_enum_values_match_binding():
    ev = _enum_values()
    assert ev["ATTN_LAYOUT_BSHD"] == attn.LAYOUTS["bshd"] and ev["ATTN_LAYOUT_BHSD"] == attn.LAYOUTS["bhsd"]
    assert ev["ATTN_ROUND_RTNE"] == attn.ROUND_MODES["rtne"]
    assert ev["ATTN_ROUND_RTNA"] == attn.ROUND_MODES["rtna"]
    assert ev["ATTN_ROUND_RTZ"] == attn.ROUND_MODES["rtz"]
    assert ev["ATTN_MASK_NONE"] == attn.MASKS["none"] and ev["ATTN_MASK_CAUSAL"] == attn.MASKS["causal"]
    assert ev["ATTN_MASK_CAUSAL_BOTTOM_RIGHT"] == attn.MASKS["causal_br"]


def test_abi_version_and_strerror():
    ev = _enum_values()
    assert attn.attn_fwd_bf16_abi_version() == int(re.search(r"ATTN_FWD_ABI_VERSION\s+(\d+)", open(HEADER).read()).group(1))
    for name, code in ev.items():
        if name.startswith("ATTN_ERR") or name == "ATTN_OK":
            assert attn.attn_fwd_bf16_strerror(code) and attn.attn_fwd_bf16_strerror(code) != "unknown status"
    assert attn.attn_fwd_bf16_strerror(12345) == "unknown status"


A, B_, C, O_ = 0x10000, 0x20000, 0x30000, 0x40000  # distinct aligned fake addresses (never dereferenced)


@pytest.mark.parametrize("args,code", [
    ((0, B_, C, O_, 1, 1, 1, 1, 0, 0), "ATTN_ERR_NULL"),
    ((A, B_, C, 0, 1, 1, 1, 1, 0, 0), "ATTN_ERR_NULL"),
    ((A, B_, C, O_, 0, 1, 1, 1, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, 1, 1, 1, 0, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, 1, -3, 1, 1, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, 1 << 40, 1 << 20, 1, 1, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, 1, (1 << 18) + 1, 1, 1, 0, 0), "ATTN_ERR_SIZE"),  # 64 K rows past 32-bit offsets
    ((A, B_, C, O_, 1, 1 << 18, 1, 1, 0, 5), "ATTN_ERR_ROUND"),       # the largest head count passes the size checks
    ((A, B_, C, O_, 1, 1, 1, 1, 2, 0), "ATTN_ERR_LAYOUT"),
    ((A, B_, C, O_, 1, 1, 1, 1, -1, 0), "ATTN_ERR_LAYOUT"),
    ((A, B_, C, O_, 1, 1, 1, 1, 0, 3), "ATTN_ERR_ROUND"),
    ((A + 2, B_, C, O_, 1, 1, 1, 1, 0, 0), "ATTN_ERR_ALIGN"),
    ((A, B_, C, O_ + 8, 1, 1, 1, 1, 0, 0), "ATTN_ERR_ALIGN"),
    ((A, B_, C, A + 128, 1, 1, 1, 1, 0, 0), "ATTN_ERR_ALIAS"),
    ((A, B_, C, B_ - 128, 1, 1, 1, 4, 0, 0), "ATTN_ERR_ALIAS"),
])
def test_argument_errors_before_any_hip_call(args, code):
    ev = _enum_values()
    assert attn.attn_fwd_bf16(*args, 0) == ev[code]


@pytest.mark.parametrize("args,code", [
    ((0, B_, C, O_, 1, 1, 1, 1, 0, 0, 1), "ATTN_ERR_NULL"),
    ((A, B_, C, O_, 1, 1, 0, 1, 0, 0, 1), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, 1, 1, 1, 1, 4, 0, 1), "ATTN_ERR_LAYOUT"),
    ((A, B_, C, O_, 1, 1, 1, 1, 0, -1, 2), "ATTN_ERR_ROUND"),
    ((A, B_ + 8, C, O_, 1, 1, 1, 1, 0, 0, 1), "ATTN_ERR_ALIGN"),
    ((A, B_, C, C, 1, 1, 1, 1, 0, 0, 2), "ATTN_ERR_ALIAS"),
    ((A, B_, C, O_, 1, 1, 1, 1, 0, 0, 3), "ATTN_ERR_MASK"),
    ((A, B_, C, O_, 1, 1, 1, 1, 0, 0, -1), "ATTN_ERR_MASK"),
])
def test_masked_argument_errors_before_any_hip_call(args, code):
    ev = _enum_values()
    assert attn.attn_fwd_bf16_masked(*args, 0) == ev[code]


@pytest.mark.parametrize("args,code", [
    ((0, B_, C, O_, 1, 4, 2, 1, 1, 0, 0, 0), "ATTN_ERR_NULL"),
    ((A, B_, C, O_, 1, 4, 0, 1, 1, 0, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, 1, 4, -2, 1, 1, 0, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, 1, 4, 3, 1, 1, 0, 0, 0), "ATTN_ERR_HEADS"),
    ((A, B_, C, O_, 1, 2, 4, 1, 1, 0, 0, 0), "ATTN_ERR_HEADS"),
    ((A, B_, C, O_, 1, 4, 2, 1, 1, 9, 0, 0), "ATTN_ERR_LAYOUT"),
    ((A, B_, C, O_, 1, 4, 2, 1, 1, 0, 5, 0), "ATTN_ERR_ROUND"),
    ((A, B_, C + 4, O_, 1, 4, 2, 1, 1, 0, 0, 0), "ATTN_ERR_ALIGN"),
    ((A, B_, C, C, 1, 4, 2, 1, 1, 0, 0, 0), "ATTN_ERR_ALIAS"),
    ((A, B_, C, O_, 1, 4, 2, 1, 1, 0, 0, 7), "ATTN_ERR_MASK"),
])
def test_gqa_argument_errors_before_any_hip_call(args, code):
    ev = _enum_values()
    assert attn.attn_fwd_bf16_gqa(*args[:4], 0, *args[4:], 0) == ev[code]


def test_gqa_alias_check_uses_the_kv_head_count():
    # k holds B*H_kv*Sk rows of 256 B: with H_kv = 1, o placed right after k does not overlap it
    ev = _enum_values()
    k_bytes = 1 * 1 * 8 * 256
    assert attn.attn_fwd_bf16_gqa(A, B_, C, B_ + k_bytes, 0, 1, 4, 1, 1, 8, 0, 0, 7, 0) == ev["ATTN_ERR_MASK"]
    assert attn.attn_fwd_bf16_gqa(A, B_, C, B_ + k_bytes - 256, 0, 1, 4, 1, 1, 8, 0, 0, 0, 0) == ev["ATTN_ERR_ALIAS"]


CQ, CK = 0x50000, 0x50100  # fake offset arrays (never dereferenced)


@pytest.mark.parametrize("args,code", [
    ((0, B_, C, O_, CQ, CK, 2, 4, 2, 10, 10, 8, 0, 0), "ATTN_ERR_NULL"),
    ((A, B_, C, O_, 0, CK, 2, 4, 2, 10, 10, 8, 0, 0), "ATTN_ERR_NULL"),
    ((A, B_, C, O_, CQ, 0, 2, 4, 2, 10, 10, 8, 0, 0), "ATTN_ERR_NULL"),
    ((A, B_, C, O_, CQ, CK, 0, 4, 2, 10, 10, 8, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, CQ, CK, 2, 4, 2, 0, 10, 8, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, CQ, CK, 2, 4, 2, 10, 0, 8, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, CQ, CK, 2, 4, 2, 10, 10, 0, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, CQ, CK, 2, 4, 2, 1 << 40, 10, 8, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, CQ, CK, 2, 4, 3, 10, 10, 8, 0, 0), "ATTN_ERR_HEADS"),
    ((A, B_, C, O_, CQ, CK, 2, 4, 2, 10, 10, 8, 3, 0), "ATTN_ERR_ROUND"),
    ((A, B_, C, O_, CQ, CK, 2, 4, 2, 10, 10, 8, 0, 4), "ATTN_ERR_MASK"),
    ((A, B_, C, O_, CQ + 2, CK, 2, 4, 2, 10, 10, 8, 0, 0), "ATTN_ERR_ALIGN"),
    ((A + 8, B_, C, O_, CQ, CK, 2, 4, 2, 10, 10, 8, 0, 0), "ATTN_ERR_ALIGN"),
    ((A, B_, C, CQ - 64, CQ, CK, 2, 4, 2, 10, 10, 8, 0, 0), "ATTN_ERR_ALIAS"),
    ((A, B_, C, A + 512, CQ, CK, 2, 4, 2, 10, 10, 8, 0, 0), "ATTN_ERR_ALIAS"),
])
def test_varlen_argument_errors_before_any_hip_call(args, code):
    ev = _enum_values()
    assert attn.attn_fwd_bf16_varlen(*args[:4], 0, *args[4:], 0) == ev[code]


L_ = 0x60000  # a fake lse array


@pytest.mark.parametrize("lse,code", [
    (L_ + 2, "ATTN_ERR_ALIGN"),   # not 4-byte aligned
    (A + 256, "ATTN_ERR_ALIAS"),  # inside q
    (O_ + 64, "ATTN_ERR_ALIAS"),  # inside o
    (O_ + 4 * 2 * 256, "ATTN_ERR_MASK"),  # just past o (4 heads x 2 rows x 256 B): fine, then the bad mask
])
def test_lse_argument_errors(lse, code):
    ev = _enum_values()
    assert attn.attn_fwd_bf16_gqa(A, B_, C, O_, lse, 1, 4, 2, 2, 8, 0, 0, 9, 0) == ev[code]
    assert attn.attn_fwd_bf16_varlen(A, B_, C, O_, lse, CQ, CK, 1, 4, 2, 2, 8, 2, 0, 9, 0) == ev[code]


def test_binding_rejects_unknown_mask_name():
    import torch

    q = torch.zeros(1, 1, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.attn_fwd(q, q, q, mask="upper")
    k3 = torch.zeros(1, 1, 3, 128, dtype=torch.bfloat16)
    q4 = torch.zeros(1, 1, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # 4 query heads over 3 K/V heads
        attn.attn_fwd(q4, k3, k3)


def test_binding_rejects_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(attn, "_lib", None)
    monkeypatch.setattr(attn, "_LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(ImportError):
        attn.load_library()


@pytest.mark.parametrize("args,code", [
    ((0, B_, C, O_, 1, 1, 1, 1, 0, 0, 0, 0), "ATTN_ERR_NULL"),
    ((A, B_, C, O_, 0, 1, 1, 1, 0, 0, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, 1, 1, 1, 1, 0, 0, 0, -1), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, 1, 1, 1, 1, 5, 0, 0, 0), "ATTN_ERR_LAYOUT"),
    ((A, B_, C, O_, 1, 1, 1, 1, 0, 7, 0, 0), "ATTN_ERR_ROUND"),
    ((A + 4, B_, C, O_, 1, 1, 1, 1, 0, 0, 0, 0), "ATTN_ERR_ALIGN"),
    ((A, B_, C, A, 1, 1, 1, 1, 0, 0, 0, 0), "ATTN_ERR_ALIAS"),
])
def test_ws_argument_errors_before_any_hip_call(args, code):
    ev = _enum_values()
    assert attn.attn_fwd_bf16_ws(*args, 0) == ev[code]


def test_workspace_size_argument_errors():
    import ctypes

    lib = attn.load_library()
    out = ctypes.c_int64(7)
    ev = _enum_values()
    assert lib.attn_fwd_bf16_workspace_size(1, 1, 1, 1, None) == ev["ATTN_ERR_NULL"]
    assert lib.attn_fwd_bf16_workspace_size(0, 1, 1, 1, ctypes.byref(out)) == ev["ATTN_ERR_SIZE"]
    assert out.value == 0
    assert lib.attn_fwd_bf16_workspace_size(1, 1, 1, -5, ctypes.byref(out)) == ev["ATTN_ERR_SIZE"]


def _plan(n_work, n_tiles, n_cu=256):
    return attn.attn_fwd_bf16_split_plan(n_work, n_tiles, n_cu)


@pytest.mark.parametrize("n_work,n_tiles,expect", [
    (816, 513, (768, 48, 5, 103)),    # B=2 H=24 Sq=4097 Sk=32771: 48 items in the last round
    (2048, 128, (2048, 0, 1, 128)),   # B=4 H=16 Sq=Sk=8192: rounds are full
    (5120, 512, (5120, 0, 1, 512)),   # B=1 H=40 Sq=Sk=32760
    (32, 1024, (0, 32, 8, 128)),      # few heads, long keys: 8 ranges each
    (2, 4, (2, 0, 1, 4)),             # too few tiles to split
    (4, 47, (0, 4, 10, 5)),           # ranges of >= 4 tiles, none empty
    (200, 1000, (200, 0, 1, 1000)),   # 200 of 256: splitting by 1 is no split
])
def test_split_plan_cases(n_work, n_tiles, expect):
    assert _plan(n_work, n_tiles) == expect


@pytest.mark.parametrize("n_work", [1, 3, 31, 100, 255, 257, 300, 511, 700, 1000, 4097])
@pytest.mark.parametrize("n_tiles", [1, 4, 7, 8, 63, 513, 2048])
def test_split_plan_invariants(n_work, n_tiles):
    n_cu = 256
    whole, items, splits, tps = _plan(n_work, n_tiles, n_cu)
    assert whole + items == n_work
    if items == 0:
        assert (splits, tps) == (1, n_tiles)
        return
    assert whole % n_cu == 0 and 0 < items < n_cu
    assert splits >= 2 and items * splits <= n_cu          # the last round fits the compute units
    assert tps >= 4 and (splits - 1) * tps < n_tiles <= splits * tps  # ranges cover the tiles, none empty


def test_split_plan_argument_errors():
    ev = _enum_values()
    import ctypes

    lib = attn.load_library()
    out = (ctypes.c_int64 * 4)()
    assert lib.attn_fwd_bf16_split_plan(1, 1, 1, None) == ev["ATTN_ERR_NULL"]
    assert lib.attn_fwd_bf16_split_plan(0, 1, 1, out) == ev["ATTN_ERR_SIZE"]
    assert lib.attn_fwd_bf16_split_plan(1, 0, 1, out) == ev["ATTN_ERR_SIZE"]
    assert lib.attn_fwd_bf16_split_plan(1, 1, 0, out) == ev["ATTN_ERR_SIZE"]


W_ = 0x70000  # a fake workspace


@pytest.mark.parametrize("args,code", [
    ((0, B_, C, O_, 0, 1, 4, 2, 1, 1, 0, 0, 1, 0, 0), "ATTN_ERR_NULL"),
    ((A, B_, C, O_, 0, 1, 4, 3, 1, 1, 0, 0, 1, 0, 0), "ATTN_ERR_HEADS"),
    ((A, B_, C, O_, 0, 1, 4, 2, 0, 1, 0, 0, 1, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, 0, 1, 4, 2, 1, 1, 2, 0, 1, 0, 0), "ATTN_ERR_LAYOUT"),
    ((A, B_, C, O_, 0, 1, 4, 2, 1, 1, 0, 3, 1, 0, 0), "ATTN_ERR_ROUND"),
    ((A, B_, C, O_, L_ + 1, 1, 4, 2, 1, 1, 0, 0, 1, 0, 0), "ATTN_ERR_ALIGN"),
    ((A, B_, C, O_, O_, 1, 4, 2, 1, 1, 0, 0, 1, 0, 0), "ATTN_ERR_ALIAS"),
    ((A, B_, C, O_, 0, 1, 4, 2, 1, 1, 0, 0, 3, 0, 0), "ATTN_ERR_MASK"),
    ((A, B_, C, O_, L_, 1, 4, 2, 1, 1, 0, 0, 1, W_, -1), "ATTN_ERR_SIZE"),  # negative workspace size
])
def test_gqa_ws_argument_errors_before_any_hip_call(args, code):
    ev = _enum_values()
    assert attn.attn_fwd_bf16_gqa_ws(*args, 0) == ev[code]


@pytest.mark.parametrize("args,code", [
    ((0, B_, C, O_, 0, 1, 4, 2, 1, 1, 0, 0, 1), "ATTN_ERR_NULL"),
    ((A, B_, C, O_, 0, 1, 4, 3, 1, 1, 0, 0, 1), "ATTN_ERR_HEADS"),
    ((A, B_, C, O_, 0, 1, 4, 2, 0, 1, 0, 0, 1), "ATTN_ERR_SIZE"),
    ((A, B_, C, O_, 0, 1, 4, 2, 1, 1, 2, 0, 1), "ATTN_ERR_LAYOUT"),
    ((A, B_, C, O_, 0, 1, 4, 2, 1, 1, 0, 3, 1), "ATTN_ERR_ROUND"),
    ((A, B_, C, O_, L_ + 1, 1, 4, 2, 1, 1, 0, 0, 1), "ATTN_ERR_ALIGN"),
    ((A, B_, C, O_, O_, 1, 4, 2, 1, 1, 0, 0, 1), "ATTN_ERR_ALIAS"),
    ((A, B_, C, O_, 0, 1, 4, 2, 1, 1, 0, 0, 3), "ATTN_ERR_MASK"),
])
def test_gqa_noalloc_argument_errors_before_any_hip_call(args, code):
    ev = _enum_values()
    assert attn.attn_fwd_bf16_gqa_noalloc(*args, 0) == ev[code]


def test_gqa_workspace_size_argument_errors():
    import ctypes

    lib = attn.load_library()
    out = ctypes.c_int64(7)
    ev = _enum_values()
    assert lib.attn_fwd_bf16_gqa_workspace_size(1, 1, 1, 1, 0, None) == ev["ATTN_ERR_NULL"]
    assert lib.attn_fwd_bf16_gqa_workspace_size(1, 0, 1, 1, 1, ctypes.byref(out)) == ev["ATTN_ERR_SIZE"]
    assert out.value == 0
    assert lib.attn_fwd_bf16_gqa_workspace_size(1, 1, 1, 1, 5, ctypes.byref(out)) == ev["ATTN_ERR_MASK"]


def _masked_plan(n_heads, Sq, Sk, mask, n_cu=256):
    return attn.attn_fwd_bf16_split_plan_masked(n_heads, Sq, Sk, attn.MASKS[mask], n_cu)


def _causal_tiles(qt, Sq, Sk, mask):
    """Key tiles q-tile qt visits, from the mask's definition: up to the last
    visible key of its last row, at least one."""
    off = Sk - Sq if mask == "causal_br" else 0
    last_row = min(Sq, 256 * qt + 256) - 1
    last_key = min(last_row + off, Sk - 1)
    return 1 if last_key < 0 else last_key // 64 + 1


@pytest.mark.parametrize("n_heads,Sq,Sk", [(48, 4097, 32771), (4, 300, 2000), (24, 512, 1280), (64, 8192, 8192),
                                           (3, 100, 100), (7, 1000, 300), (10, 256, 64 * 40)])
def test_masked_plan_without_mask_is_the_plain_plan(n_heads, Sq, Sk):
    n_qt = -(-Sq // 256)
    assert _masked_plan(n_heads, Sq, Sk, "none") == _plan(n_heads * n_qt, -(-Sk // 64))


@pytest.mark.parametrize("n_heads,Sq,Sk,mask,expect", [
    (48, 4097, 32771, "causal_br", (768, 48, 5, 103)),  # prefill after 28674 cached keys: items nearly equal
    (48, 4097, 32771, "causal", (816, 0, 1, 65)),      # top-left: q-tiles see 4 .. 65 tiles, no split
    (64, 8192, 8192, "causal", (2048, 0, 1, 128)),
    (24, 512, 1280, "causal_br", (0, 48, 5, 4)),        # q-tiles see 16 and 20 tiles: 5 ranges of the longest
    (4, 300, 2000, "causal_br", (0, 8, 8, 4)),
    (4, 2000, 300, "causal_br", (32, 0, 1, 5)),         # Sq > Sk: the first q-tiles see no key
    (4, 16384, 16384, "causal", (0, 256, 2, 128)),      # one round of unequal items (4 .. 256 tiles): all cut in 2
    (2, 8192, 8192, "causal", (0, 64, 8, 16)),          # 64 items: 8 ranges each
    (1, 1000, 1000, "causal", (0, 4, 4, 4)),            # ranges of at least 4 tiles of the longest item
    (16, 8192, 8192, "causal", (512, 0, 1, 128)),       # two rounds: longest first, no split
])
def test_masked_plan_cases(n_heads, Sq, Sk, mask, expect):
    assert _masked_plan(n_heads, Sq, Sk, mask) == expect


@pytest.mark.parametrize("mask", ["causal", "causal_br"])
@pytest.mark.parametrize("n_heads", [1, 3, 24, 100, 257])
@pytest.mark.parametrize("Sq,Sk", [(100, 100), (300, 2000), (512, 1280), (1000, 30000), (4097, 32771), (2000, 300),
                                   (8192, 8192)])
def test_masked_plan_invariants(mask, n_heads, Sq, Sk):
    n_cu = 256
    n_qt = -(-Sq // 256)
    whole, items, splits, tps = _masked_plan(n_heads, Sq, Sk, mask, n_cu)
    tiles = [_causal_tiles(qt, Sq, Sk, mask) for qt in range(n_qt)]
    n_work = n_heads * n_qt
    assert whole + items == n_work
    if items == 0:
        assert splits == 1
        # nothing split: nearly equal items filling whole rounds, unequal ones over several
        # rounds, or too few tiles to cut
        assert (4 * min(tiles) >= 3 * max(tiles)) or n_work > n_cu or max(tiles) < 8
        return
    assert splits >= 2 and tps >= 4 and (splits - 1) * tps < max(tiles) <= splits * tps
    if 4 * min(tiles) >= 3 * max(tiles):  # nearly equal items: only the partly idle last round
        assert whole % n_cu == 0 and 0 < items < n_cu and items * splits <= n_cu
    else:  # unequal items in one round: all of them, up to twice as many workgroups as CUs
        assert n_work <= n_cu and whole == 0 and items == n_work
        assert splits <= 8 and n_work * splits <= 2 * n_cu


def test_masked_plan_argument_errors():
    import ctypes

    ev = _enum_values()
    lib = attn.load_library()
    out = (ctypes.c_int64 * 4)()
    assert lib.attn_fwd_bf16_split_plan_masked(1, 1, 1, 0, 1, None) == ev["ATTN_ERR_NULL"]
    assert lib.attn_fwd_bf16_split_plan_masked(0, 1, 1, 0, 1, out) == ev["ATTN_ERR_SIZE"]
    assert lib.attn_fwd_bf16_split_plan_masked(1, 1, 0, 0, 1, out) == ev["ATTN_ERR_SIZE"]
    assert lib.attn_fwd_bf16_split_plan_masked(1, 1, 1, 0, 0, out) == ev["ATTN_ERR_SIZE"]
    assert lib.attn_fwd_bf16_split_plan_masked(1, 1, 1, 3, 1, out) == ev["ATTN_ERR_MASK"]


P_ = 0x80000  # a fake fp32 partial output (4 heads x 2 rows x 512 B = 4 KiB)
PL = 0x90000  # a fake partial lse


@pytest.mark.parametrize("args,code", [
    # q, k, v, o_part, lse_part, B, H, H_kv, Sq, Sk, key_offset, Sk_total, layout, mask
    ((0, B_, C, P_, PL, 1, 4, 2, 2, 8, 0, 8, 0, 0), "ATTN_ERR_NULL"),
    ((A, B_, C, 0, PL, 1, 4, 2, 2, 8, 0, 8, 0, 0), "ATTN_ERR_NULL"),
    ((A, B_, C, P_, 0, 1, 4, 2, 2, 8, 0, 8, 0, 0), "ATTN_ERR_NULL"),
    ((A, B_, C, P_, PL, 1, 4, 3, 2, 8, 0, 8, 0, 0), "ATTN_ERR_HEADS"),
    ((A, B_, C, P_, PL, 1, 4, 2, 2, 8, -1, 8, 0, 0), "ATTN_ERR_SIZE"),     # shard before the first key
    ((A, B_, C, P_, PL, 1, 4, 2, 2, 8, 1, 8, 0, 0), "ATTN_ERR_SIZE"),      # shard past the last key
    ((A, B_, C, P_, PL, 1, 4, 2, 2, 8, 0, 1 << 31, 0, 0), "ATTN_ERR_SIZE"),
    ((A, B_, C, P_, PL, 1, 4, 2, 2, 8, 0, 8, 3, 0), "ATTN_ERR_LAYOUT"),
    ((A, B_, C, P_ + 8, PL, 1, 4, 2, 2, 8, 0, 8, 0, 0), "ATTN_ERR_ALIGN"),
    ((A, B_, C, P_, PL + 2, 1, 4, 2, 2, 8, 0, 8, 0, 0), "ATTN_ERR_ALIGN"),
    ((A, B_, C, P_, P_ + 2048, 1, 4, 2, 2, 8, 0, 8, 0, 0), "ATTN_ERR_ALIAS"),  # lse inside the fp32 rows
    ((A, B_, C, A - 2048, PL, 1, 4, 2, 2, 8, 0, 8, 0, 0), "ATTN_ERR_ALIAS"),  # fp32 rows (2x q's bytes) reach q
    ((A, B_, C, P_, PL, 1, 4, 2, 2, 8, 0, 8, 0, 4), "ATTN_ERR_MASK"),
    ((A, B_, C, P_, PL, 1, 4, 2, 2, 8, 2, 10, 0, 4), "ATTN_ERR_MASK"),    # a shard in the middle passes the checks
])
def test_partial_argument_errors_before_any_hip_call(args, code):
    ev = _enum_values()
    assert attn.attn_fwd_bf16_partial(*args, 0) == ev[code]


@pytest.mark.parametrize("args,code", [
    # o_parts, lse_parts, n_parts, o, lse, B, H, Sq, layout, round_mode
    ((0, PL, 2, O_, 0, 1, 4, 2, 0, 0), "ATTN_ERR_NULL"),
    ((P_, 0, 2, O_, 0, 1, 4, 2, 0, 0), "ATTN_ERR_NULL"),
    ((P_, PL, 2, 0, 0, 1, 4, 2, 0, 0), "ATTN_ERR_NULL"),
    ((P_, PL, 0, O_, 0, 1, 4, 2, 0, 0), "ATTN_ERR_SIZE"),
    ((P_, PL, 2, O_, 0, 1, 0, 2, 0, 0), "ATTN_ERR_SIZE"),
    ((P_, PL, 2, O_, 0, 1 << 40, 1 << 18, 2, 0, 0), "ATTN_ERR_SIZE"),
    ((P_, PL, 2, O_, 0, 1, 4, 2, 2, 0), "ATTN_ERR_LAYOUT"),
    ((P_, PL, 2, O_, 0, 1, 4, 2, 0, 3), "ATTN_ERR_ROUND"),
    ((P_ + 4, PL, 2, O_, 0, 1, 4, 2, 0, 0), "ATTN_ERR_ALIGN"),
    ((P_, PL, 2, O_ + 8, 0, 1, 4, 2, 0, 0), "ATTN_ERR_ALIGN"),
    ((P_, PL, 2, O_, L_ + 1, 1, 4, 2, 0, 0), "ATTN_ERR_ALIGN"),
    ((P_, PL, 2, P_ + 4096, 0, 1, 4, 2, 0, 0), "ATTN_ERR_ALIAS"),     # o over the second part
    ((P_, PL, 2, O_, PL + 32, 1, 4, 2, 0, 0), "ATTN_ERR_ALIAS"),      # lse over the second part's lse
    ((P_, PL, 2, O_, O_ + 64, 1, 4, 2, 0, 0), "ATTN_ERR_ALIAS"),      # lse inside o
])
def test_merge_argument_errors_before_any_hip_call(args, code):
    ev = _enum_values()
    assert attn.attn_fwd_bf16_merge(*args, 0) == ev[code]
