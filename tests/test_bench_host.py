"""bench.py's host logic, without a GPU: the FLOP count of each workload (the
visible (query, key) pairs against a brute-force count), the code hash that
ties the committed traffic counters to a kernel version, the traffic reader,
and the refusal of more than one GPU."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from bf16_forward_attention_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _pairs_brute(Sq, Sk, mask):
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    if mask == "none":
        return Sq * Sk
    off = 0 if mask == "causal" else Sk - Sq
    return int(np.sum(j <= i + off))


@pytest.mark.parametrize("mask", ["none", "causal", "causal_br"])
@pytest.mark.parametrize("Sq,Sk", [(1, 1), (7, 300), (300, 7), (257, 257), (1000, 64), (64, 1000)])
def test_workload_flops_counts_visible_pairs(mask, Sq, Sk):
    wl = synth.Workload("t", 2, 3, Sq, Sk, "bshd", ("rtne",), mask=mask)
    assert bench.workload_flops(wl) == 4 * 128 * 2 * 3 * _pairs_brute(Sq, Sk, mask)


def test_named_workloads_flops():
    assert bench.workload_flops(synth.WORKLOADS["self8k"]) == 4 * 128 * 4 * 16 * 8192 * 8192
    # causal at Sq = Sk: S(S+1)/2 pairs per head
    assert bench.workload_flops(synth.WORKLOADS["self8k_causal"]) == 4 * 128 * 4 * 16 * 8192 * 8193 // 2
    wl = synth.WORKLOADS["prefill_br"]
    assert bench.workload_flops(wl) == 4 * 128 * wl.B * wl.H * _pairs_brute(wl.Sq, wl.Sk, "causal_br")


def test_varlen_pairs_match_a_brute_force_count():
    wl = synth.VARLEN_WORKLOADS["varlen_mix"]
    got = bench.varlen_visible_pairs(wl)
    expect = [_pairs_brute(sq, sk, wl.mask) for sq, sk in zip(wl.lengths_q, wl.lengths_k)]
    assert got.tolist() == expect and sum(wl.lengths_q) == 77048


def test_code_hash_ignores_comments_and_follows_code(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "bf16_forward_attention_amd", "csrc", "attn_fwd.hip")
    text = open(src).read()
    base = bench.kernel_code_sha256()
    fake_root = tmp_path / "r"
    (fake_root / "bf16_forward_attention_amd" / "csrc").mkdir(parents=True)
    dst = fake_root / "bf16_forward_attention_amd" / "csrc" / "attn_fwd.hip"
    monkeypatch.setattr(bench, "ROOT", str(fake_root))
    dst.write_text("// a new comment line\n\n" + text.replace("constexpr int BM = 256;", "constexpr int BM = 256;  // rows"))
    assert bench.kernel_code_sha256() == base
    dst.write_text(text.replace("constexpr int BM = 256;", "constexpr int BM = 128;"))
    assert bench.kernel_code_sha256() != base


def test_traffic_summary_is_used_only_for_its_kernel(monkeypatch):
    got = bench.measured_traffic("self8k")
    if got is not None:  # counters of this kernel version: about Q+K+V+O once
        assert abs(got - 536_870_912) < 0.01 * 536_870_912
    monkeypatch.setattr(bench, "kernel_code_sha256", lambda: "0" * 64)
    assert bench.measured_traffic("self8k") is None
    assert bench.measured_traffic("no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in (r.stdout + r.stderr)


def _smi_reply(mhz, power=None, wrap=True):
    clock = {f"gfx_{i}": {"clk": {"value": c, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
                          "max_clk": {"value": 2400, "unit": "MHz"}} for i, c in enumerate(mhz)}
    clock["mem_0"] = {"clk": {"value": 2000, "unit": "MHz"}}
    g = {"gpu": 0, "clock": clock}
    if power is not None:
        g["power"] = {"socket_power": {"value": power, "unit": "W"}, "gfx_voltage": "N/A"}
    return {"gpu_data": [g]} if wrap else [g]


def test_smi_metric_parsing():
    mhz = [1815, 1720, 1795, 1718, 1804, 1713, 1769, 1688, 1700, 1701, 1702]
    res = bench.parse_smi_metric(_smi_reply(mhz, power=1380))
    # XCDs in index order (gfx_10 after gfx_9), memory clock left out
    assert res["gfx_mhz_per_xcd"] == mhz
    assert res["gfx_mhz_mean"] == round(sum(mhz) / len(mhz), 1)
    assert res["gfx_mhz_max"] == 2400 and res["socket_power_w"] == 1380
    assert "socket_power_w" not in bench.parse_smi_metric(_smi_reply([100, 200], wrap=False))
    # no reply, no GPU, two GPUs (ambiguous), a clock field that is not a number
    assert bench.parse_smi_metric(None) is None
    assert bench.parse_smi_metric({"gpu_data": []}) is None
    two = _smi_reply([1700])
    two["gpu_data"].append(dict(two["gpu_data"][0], gpu=1))
    assert bench.parse_smi_metric(two) is None
    assert bench.parse_smi_metric(_smi_reply(["N/A"])) is None


def test_smi_index_by_pci_address():
    listing = [{"gpu": 0, "bdf": "0000:05:00.0"}, {"gpu": 1, "bdf": "0000:75:00.0"}]
    assert bench.smi_index("0000:75:00", listing) == 1
    assert bench.smi_index("0000:05:00", {"gpu_data": listing}) == 0
    assert bench.smi_index("0000:99:00", listing) is None
    assert bench.smi_index("0000:05:00", None) is None


def test_amd_smi_missing_tool(monkeypatch):
    monkeypatch.setattr(bench.shutil, "which", lambda name: None)
    monkeypatch.setattr(bench.subprocess, "run", lambda *a, **k: (_ for _ in ()).throw(OSError("no such file")))
    assert bench.amd_smi("list") is None


def test_profiler_detection(monkeypatch):
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/rocprofiler-sdk/librocprofiler-sdk-tool.so:/x/lib.so")
    assert bench.under_profiler()
    monkeypatch.setenv("LD_PRELOAD", "/usr/lib/libother.so")
    assert not bench.under_profiler()
    monkeypatch.delenv("LD_PRELOAD")
    assert not bench.under_profiler()


def test_sweep_covers_the_long_configurations_and_their_modes():
    names = {(n, m) for n, m in bench.SWEEP}
    assert {("long128k", m) for m in ("rtne", "rtna", "rtz")} <= names
    assert ("cross_odd", "rtz") in names and ("dit_stress", "rtna") in names
    for n, m in bench.SWEEP:
        wl = synth.WORKLOADS[n]
        assert m in wl.modes and max(wl.Sq, wl.Sk) >= 8192


def test_sweep_parity_rows():
    # the long-context rows come from its own checked subset; the stressed workload's sample holds
    # x64-scaled rows and rows of every head with a K special
    wl = synth.WORKLOADS["long128k"]
    inp = synth.Inputs(wl, None, None, None)
    rows = bench.sweep_parity_rows(inp)
    checked = set(synth.checked_rows(wl))
    assert len(rows) >= 128 and set(rows) <= checked
    wl = synth.WORKLOADS["dit_stress"]
    inp = synth.Inputs(wl, None, None, None, synth.scaled_row_list(wl), synth.special_list(wl))
    rows = set(bench.sweep_parity_rows(inp))
    scaled = {(f // (wl.H * wl.Sq), (f // wl.Sq) % wl.H, f % wl.Sq) for f in inp.scaled_rows[:16]}
    assert scaled <= rows
    for _, b, h, _, _ in inp.specials:
        assert sum(1 for r in rows if r[:2] == (b, h)) >= 8
    assert all(0 <= i < wl.Sq for _, _, i in rows)


def test_power_reference_is_the_headline_on_zero_operands():
    assert len(bench.POWER_REFERENCE) == 1
    name, mode = bench.POWER_REFERENCE[0]
    wl, head = synth.WORKLOADS[name], synth.WORKLOADS["self8k"]
    assert wl.zero_kv and mode in wl.modes and (name, mode) not in bench.SWEEP
    assert (wl.B, wl.H, wl.Sq, wl.Sk, wl.layout, wl.mask) == (head.B, head.H, head.Sq, head.Sk, head.layout, head.mask)
