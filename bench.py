#!/usr/bin/env python3
"""Benchmark of the fused bf16 forward attention on one MI355X.

A step is one call of the library over the whole workload (every query row of
every head), inputs resident in HBM: attn_fwd_bf16_ws with a preallocated
workspace when the shape splits its key ranges (then the step is both of its
kernels; attn_fwd_bf16_gqa_ws for the causal and grouped-query workloads),
attn_fwd_bf16_gqa (grouped) or attn_fwd_bf16_masked (causal) for those that
do not split, attn_fwd_bf16 otherwise.  Default workload: self-attention B=4, H=16, Sq=Sk=8192, d=128,
BSHD, RTNE.  Prints one JSON line:

  value      forward TFLOP/s, 4*128 FLOPs per visible (query, key) pair (all
             B*H*Sq*Sk of them without a mask) / mean step time
  roofline   the kernel against MI355X's dense bf16 MFMA peak, with the
             per-launch duration measured by HIP events on the launch stream
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload's
             rows, timed on this host's cores (a reported baseline only)
  parity     rows of the timed output, taken from those the CPU baseline
             computed, checked against them under the row-scaled 2-ULP gate
  clock      the shader clock of each XCD and the socket power (amd-smi) during
             about 4 s more of the same launches right after the timed region, and
             the rate over the last 2 s of them (sustained_tflops)
  env        ROCm and torch versions, the device, the hipcc flags of the build and the
             hash of the kernel source (the one the profiles/ summaries name)
  sweep      (with the default workload, or --sweep; under rocprofv3 only with --sweep)
             the other configurations of 8K and longer, each timed alone the same way
             after the headline: the 128K long-context workload in all three rounding
             modes, the 4097 x 32771 cross-attention and the stressed 32760 x 32760
             workload, each with its rate, share of the peak, clock and a parity sample
             against the oracle
  power_reference  (with the sweep) the headline's shapes and instructions on K = V = 0,
             timed the same way: not a benchmark workload, a reference for how far the
             arithmetic on random data lowers the clock under the power limit

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--mode rtne|rtna|rtz] [--no-cpu-baseline] [--cpu-seconds S] [--no-split] [--no-clock]
       [--sweep | --no-sweep] [--sweep-seconds S]
"""
from __future__ import annotations

import argparse
import json
import os
import shutil
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MI355X bf16 MFMA peak, d=128, S=8K–128K"
# MI355X dense bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU (the published 2.5 PFLOP/s)
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def amd_smi(*args):
    """One ``amd-smi ... --json`` query, parsed; None where the tool is missing or fails."""
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    try:
        out = subprocess.run([exe, *args, "--json"], capture_output=True, text=True, timeout=10).stdout
        starts = [i for i in (out.find("{"), out.find("[")) if i >= 0]
        return json.JSONDecoder().raw_decode(out[min(starts):])[0] if starts else None
    except (OSError, subprocess.SubprocessError, ValueError):
        return None


def _gpu_entries(obj):
    if isinstance(obj, dict):
        obj = obj.get("gpu_data", [obj])
    return [g for g in obj if isinstance(g, dict)] if isinstance(obj, list) else []


def smi_index(bdf: str, listing) -> int | None:
    """amd-smi's index of the GPU at PCI address ``bdf`` ("dddd:bb:dd"), from ``amd-smi list``."""
    for g in _gpu_entries(listing):
        if str(g.get("bdf", "")).lower().startswith(bdf.lower()) and "gpu" in g:
            return int(g["gpu"])
    return None


def parse_smi_metric(obj) -> dict | None:
    """Shader clock per XCD (MHz, the ``gfx_N`` entries) and socket power (W) of the one GPU in an
    ``amd-smi metric -c -p`` reply."""
    gpus = _gpu_entries(obj)
    if len(gpus) != 1:
        return None
    g = gpus[0]
    clocks = g.get("clock", {})
    xcd = sorted((k for k in clocks if k.startswith("gfx_") and k[4:].isdigit()), key=lambda k: int(k[4:]))
    mhz = []
    for k in xcd:
        clk = clocks[k].get("clk") if isinstance(clocks[k], dict) else None
        if isinstance(clk, dict) and isinstance(clk.get("value"), (int, float)):
            mhz.append(clk["value"])
    if not mhz:
        return None
    res = {"gfx_mhz_per_xcd": mhz, "gfx_mhz_mean": round(sum(mhz) / len(mhz), 1)}
    top = clocks[xcd[0]].get("max_clk")
    if isinstance(top, dict) and isinstance(top.get("value"), (int, float)):
        res["gfx_mhz_max"] = top["value"]
    power = g.get("power")
    power = power.get("socket_power") if isinstance(power, dict) else None
    if isinstance(power, dict) and isinstance(power.get("value"), (int, float)):
        res["socket_power_w"] = power["value"]
    return res


def clock_sample(step, launch_ms: float, stream, dev, seconds: float = 4.0) -> dict:
    """The clock under the timed load.  amd-smi reports a clock averaged over a window of about a
    second, so the same launches run on for ``seconds`` more (outside the timed region; they rewrite
    the same output) in chunks of about 0.4 s, one chunk always queued ahead, with a reading after
    each chunk is queued.  Returns the last reading, the mean clock of every reading in order, and
    the mean launch time over the second half of the chunks (the rate once the clock has settled)."""
    import torch

    p = torch.cuda.get_device_properties(dev)
    idx = smi_index(f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}", amd_smi("list"))
    sel = ["-g", str(idx)] if idx is not None else []
    per_chunk = max(1, int(400.0 / max(launch_ms, 1e-3)))
    n_chunks = max(2, int(round(seconds * 1e3 / (per_chunk * launch_ms))))

    spans = []

    def chunk():
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(per_chunk):
            step()
        b.record(stream)
        spans.append((a, b))
        return b

    pending = [chunk()]
    series, last, under_load, asking = [], None, False, True
    for _ in range(n_chunks - 1):
        pending.append(chunk())
        if asking:
            reply = parse_smi_metric(amd_smi("metric", *sel, "-c", "-p"))
            under_load = not pending[-1].query()
            if reply is None:
                asking = False  # no tool, no clock in its reply, or a time-out: ask no more
            else:
                last = reply
                series.append(reply["gfx_mhz_mean"])
        pending.pop(0).synchronize()
    torch.cuda.synchronize()
    settled = spans[len(spans) // 2:]
    sustained_ms = sum(a.elapsed_time(b) for a, b in settled) / (per_chunk * len(settled))
    if last is None:
        return {"unavailable": "amd-smi gave no clock for this GPU", "sustained_launch_ms": round(sustained_ms, 4)}
    last["under_load"] = under_load
    last["gfx_mhz_mean_series"] = series
    last["launches"] = per_chunk * n_chunks
    last["sustained_launch_ms"] = round(sustained_ms, 4)
    static = _gpu_entries(amd_smi("static", *sel, "--asic"))
    if len(static) == 1 and isinstance(static[0].get("asic"), dict):
        last["market_name"] = static[0]["asic"].get("market_name")
    # the dense bf16 peak at the clock the XCDs ran at
    last["mfma_peak_at_clock_tflops"] = round(p.multi_processor_count * last["gfx_mhz_mean"] * 1e6 * 4096 / 1e12, 1)
    return last


def under_profiler() -> bool:
    """True when rocprofv3 has preloaded its library into this process: the clock sample is then
    left out, so that no amd-smi child runs under the profiler and the traced launches are the
    timed ones."""
    return "rocprofiler" in os.environ.get("LD_PRELOAD", "")


def run_env(dev) -> dict:
    """Versions and build flags the figures were taken with."""
    import torch

    from bf16_forward_attention_amd import build

    p = torch.cuda.get_device_properties(dev)
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        rocm = None
    return {"rocm": rocm, "torch": torch.__version__, "hip": torch.version.hip, "device": p.name,
            "arch": p.gcnArchName, "cus": p.multi_processor_count,
            "hipcc_flags": " ".join(build.HIPCC_FLAGS), "kernel_code_sha256": kernel_code_sha256()}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="self8k")
    p.add_argument("--mode", default=None, help="rounding mode (default: the workload's first)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-split", action="store_true", help="always run single-pass (no key-range split)")
    p.add_argument("--no-clock", action="store_true",
                   help="leave out the clock sample (its ~4 s of extra launches and the amd-smi queries); "
                        "it is left out by itself under rocprofv3")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle wall time for the sample")
    p.add_argument("--parity-rows", type=int, default=256)
    p.add_argument("--sweep", dest="sweep", action="store_true", default=None,
                   help="also time the other configurations of 8K and longer (default: with the default workload)")
    p.add_argument("--no-sweep", dest="sweep", action="store_false")
    p.add_argument("--sweep-seconds", type=float, default=1.5, help="timed launches per sweep configuration")
    p.add_argument("--sweep-warmup", type=int, default=3)
    p.add_argument("--sweep-clock-seconds", type=float, default=3.0)
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="also run one device-to-device copy of this many MiB (a reference kernel of known "
                        "traffic for the FETCH_SIZE/WRITE_SIZE counters)")
    return p.parse_args()


def head_rows(wl, n, b, h, stream):
    """``n`` seeded distinct query rows of head (b, h)."""
    from bf16_forward_attention_amd import synth

    idx = synth.floyd_sample(wl.seed, synth.TID_SUBSET, wl.Sq, min(n, wl.Sq), stream=stream)
    return [(b, h, i) for i in idx]


def visible_keys(wl, rows_i):
    """Keys each query row attends to: all Sk, or j <= i + off under a causal mask."""
    i = np.asarray(rows_i, dtype=np.int64)
    if wl.mask == "none":
        return np.full(i.shape, wl.Sk, dtype=np.int64)
    off = 0 if wl.mask == "causal" else wl.Sk - wl.Sq
    return np.clip(i + off + 1, 0, wl.Sk)


def workload_flops(wl) -> float:
    return 4.0 * 128 * wl.B * wl.H * float(visible_keys(wl, np.arange(wl.Sq)).sum())


def cpu_baseline(inp, target_s, n_parity):
    """Time the oracle, as it stands, on a bounded row sample of this workload.

    A short probe (rows of one head) sizes the sample to about ``target_s``
    seconds; the timed sample then takes rows from consecutive heads.  Returns
    the baseline record and, for the parity check of the GPU output, up to
    ``n_parity`` of the timed rows (evenly spread) with the oracle's outputs
    for them: the oracle runs only here.
    """
    import oracle

    wl = inp.wl
    threads = oracle.default_threads()
    # two probes on one head: the difference is the marginal cost of a row,
    # the rest is the per-head decode of K and V
    times = []
    for n_probe in (2 * threads, 6 * threads):
        probe = head_rows(wl, n_probe, 0, 0, stream=1 << 20)
        t0 = time.perf_counter()
        oracle.attn_rows(inp.q, inp.k, inp.v, wl.layout, probe, threads, mask=wl.mask)
        times.append((len(probe), time.perf_counter() - t0))
    (n1, t1), (n2, t2) = times
    per_row = max((t2 - t1) / max(n2 - n1, 1), 1e-9)
    per_head_fixed = max(t1 - n1 * per_row, 0.0)
    per_head = min(wl.Sq, 1024)
    n = int(min(wl.B * wl.H * wl.Sq, max(threads, target_s / (per_row + per_head_fixed / per_head))))
    per_head = min(wl.Sq, max(per_head, -(-n // (wl.B * wl.H))))
    rows = []
    bh = 0
    while len(rows) < n and bh < wl.B * wl.H:
        take = min(per_head, n - len(rows))
        rows += head_rows(wl, take, bh // wl.H, bh % wl.H, stream=(1 << 21) + bh)
        bh += 1
    t0 = time.perf_counter()
    ex, rd = oracle.attn_rows(inp.q, inp.k, inp.v, wl.layout, rows, threads, mask=wl.mask)
    dt = time.perf_counter() - t0
    pairs = int(visible_keys(wl, [i for _, _, i in rows]).sum())
    flops = 4.0 * pairs * 128
    keys = f"all {wl.Sk} keys each" if wl.mask == "none" else f"{pairs} visible (query, key) pairs"
    record = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
              "sample": f"{len(rows)} seeded query rows from {bh} heads of {wl.name} ({keys}, "
                        f"fp64 with 3 roundings), {dt:.2f} s"}
    idx = np.unique(np.linspace(0, len(rows) - 1, min(n_parity, len(rows))).astype(np.int64))
    return record, [rows[i] for i in idx], ex[idx], rd[idx]


def kernel_code_sha256() -> str:
    """SHA-256 of the kernel source's code: '//' comments, trailing blanks and
    empty lines removed (the file has no block comments and no '//' in a
    string), so that an edit of a comment does not disown the counters."""
    import hashlib
    import re

    path = os.path.join(ROOT, "bf16_forward_attention_amd", "csrc", "attn_fwd.hip")
    lines = []
    with open(path) as f:
        for line in f:
            code = re.sub(r"//.*$", "", line.rstrip("\n")).rstrip()
            if code.strip():
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary.

    The summary (profiles/attn_fwd_traffic_<workload>.txt) records the two
    counters per dispatch, the scale factors a plain copy of known size gave
    them, and the SHA-256 of the kernel code they were taken on
    (kernel_code_sha256); a summary of another kernel version gives None.
    """
    path = os.path.join(ROOT, "profiles", f"attn_fwd_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_code_sha256") != kernel_code_sha256():
        return None
    fetch = float(kv["fetch_size_kib_per_launch"]) * float(kv["copy_fetch_scale"])
    write = float(kv["write_size_kib_per_launch"]) * float(kv["copy_write_scale"])
    return int(round((fetch + write) * 1024))


def make_step(attn, wl, mode, q, k, v, o, stream, dev, no_split):
    """The call one step makes for workload ``wl`` in ``mode`` on resident tensors:
    attn_fwd_bf16_ws / attn_fwd_bf16_gqa_ws with a preallocated workspace where the shape
    splits its key ranges, attn_fwd_bf16_gqa (grouped), attn_fwd_bf16_masked (causal) or
    attn_fwd_bf16 otherwise.  Returns (step, description, workspace bytes, workspace)."""
    import torch

    masked = wl.mask != "none"
    grouped = wl.kv_heads != wl.H
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    if no_split:
        ws_bytes = 0
    elif masked or grouped:
        ws_bytes = attn.attn_fwd_bf16_gqa_workspace_size(wl.B, wl.H, wl.Sq, wl.Sk, attn.MASKS[wl.mask])
    else:
        ws_bytes = attn.attn_fwd_bf16_workspace_size(wl.B, wl.H, wl.Sq, wl.Sk)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    args_c = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), wl.B, wl.H, wl.Sq, wl.Sk,
              attn.LAYOUTS[wl.layout], attn.ROUND_MODES[mode])
    if ws_bytes > 0 and (masked or grouped):
        whole, items, splits, tps = attn.attn_fwd_bf16_split_plan_masked(wl.B * wl.H, wl.Sq, wl.Sk,
                                                                         attn.MASKS[wl.mask], n_cu)
        entry = (f"attn_fwd_bf16_gqa_ws(H_kv={wl.kv_heads}, {wl.mask}): {whole} work items whole, {items} split "
                 f"into {splits} key ranges (of up to {tps} tiles), {ws_bytes} B workspace")
    elif ws_bytes > 0:
        whole, items, splits, tps = attn.attn_fwd_bf16_split_plan(wl.B * wl.H * -(-wl.Sq // 256), -(-wl.Sk // 64),
                                                                  n_cu)
        entry = (f"attn_fwd_bf16_ws: {whole} work items whole, {items} split into {splits} key ranges of "
                 f"{tps} tiles, {ws_bytes} B workspace")
    elif grouped:
        entry = f"attn_fwd_bf16_gqa(H_kv={wl.kv_heads}, {wl.mask})"
    elif masked:
        entry = f"attn_fwd_bf16_masked({wl.mask})"
    else:
        entry = "attn_fwd_bf16"

    def step():
        if ws_bytes > 0 and (masked or grouped):
            st = attn.attn_fwd_bf16_gqa_ws(args_c[0], args_c[1], args_c[2], args_c[3], 0, wl.B, wl.H, wl.kv_heads,
                                           wl.Sq, wl.Sk, args_c[8], args_c[9], attn.MASKS[wl.mask], ws.data_ptr(),
                                           ws_bytes, stream.cuda_stream)
        elif ws_bytes > 0:
            st = attn.attn_fwd_bf16_ws(*args_c, ws.data_ptr(), ws_bytes, stream.cuda_stream)
        elif grouped:
            st = attn.attn_fwd_bf16_gqa(args_c[0], args_c[1], args_c[2], args_c[3], 0, wl.B, wl.H, wl.kv_heads, wl.Sq,
                                        wl.Sk, args_c[8], args_c[9], attn.MASKS[wl.mask], stream.cuda_stream)
        elif masked:
            st = attn.attn_fwd_bf16_masked(*args_c, attn.MASKS[wl.mask], stream.cuda_stream)
        else:
            st = attn.attn_fwd_bf16(*args_c, stream.cuda_stream)
        if st != 0:
            raise attn.AttnError(st)

    return step, entry, ws_bytes, ws


def time_launches(step, stream, steps):
    """``steps`` launches, each bracketed by HIP events on the launch stream: (ms per step over
    the whole region, per-launch times in ms)."""
    import torch

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    return starts[0].elapsed_time(ends[-1]) / steps, per


# The configurations of sequence length 8K and longer besides the headline one, timed after it
# in the same run: the long-context workload in every rounding mode, the cross-attention with odd
# lengths and the stressed diffusion-transformer-like workload.
SWEEP = (("long128k", "rtne"), ("long128k", "rtna"), ("long128k", "rtz"), ("cross_odd", "rtz"),
         ("dit_stress", "rtna"))
# timed after the sweep and reported apart from it: the headline's shapes and instructions on zero K and V,
# a reference for how much the arithmetic on random data lowers the clock under the power limit
POWER_REFERENCE = (("self8k_zero_kv", "rtne"),)
POWER_REFERENCE_NOTE = ("not a benchmark workload: self8k with K = V = 0 (every output 0), the same "
                        "instructions on operands that barely switch; set its clock and rate against "
                        "the headline's")


def sweep_parity_rows(inp, n=128):
    """Rows the sweep's parity sample checks: the workload's own checked subset where it has one,
    else seeded rows of every head plus each head's last row; the stressed workload adds some of
    its x64-scaled rows and rows of the heads with K specials."""
    from bf16_forward_attention_amd import synth

    wl = inp.wl
    n_heads = wl.B * wl.H
    per = max(1, n // n_heads)
    rows = set()
    for bh in range(n_heads):
        b, h = divmod(bh, wl.H)
        if wl.checked_rows_per_head:
            subset = synth.floyd_sample(wl.seed, synth.TID_SUBSET, wl.Sq, wl.checked_rows_per_head, stream=bh)
            rows.update((b, h, i) for i in subset[:per])
        else:
            rows.update(head_rows(wl, per, b, h, stream=(1 << 22) + bh))
            rows.add((b, h, wl.Sq - 1))
    for f in inp.scaled_rows[:16]:
        rows.add((f // (wl.H * wl.Sq), (f // wl.Sq) % wl.H, f % wl.Sq))
    for _, b, h, _, _ in inp.specials:
        rows.update(head_rows(wl, 8, b, h, stream=(1 << 23) + b * wl.H + h))
    return sorted(rows)


def run_sweep(args, dev, configs=SWEEP):
    """Time each configuration of ``configs`` on its own (inputs resident, the same launch protocol
    as the headline), with the clock under it and a parity sample of its output against the
    oracle."""
    import torch

    import bf16_forward_attention_amd as attn
    import oracle
    from bf16_forward_attention_amd import synth
    from tests.gate import gate

    stream = torch.cuda.current_stream(dev)
    out = []
    loaded = None
    for name, mode in configs:
        wl = synth.WORKLOADS[name]
        if loaded is None or loaded[0].wl.name != name:
            loaded = None
            torch.cuda.empty_cache()
            t0 = time.perf_counter()
            inp = synth.generate(wl)
            t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            loaded = (inp, t(inp.q), t(inp.k), t(inp.v))
            log(f"[bench] sweep: generated {name} in {time.perf_counter() - t0:.1f} s")
            rows = sweep_parity_rows(inp)
            t0 = time.perf_counter()
            ex, rd = oracle.attn_rows(inp.q, inp.k, inp.v, wl.layout, rows, mask=wl.mask)
            log(f"[bench] sweep: oracle on {len(rows)} rows of {name} in {time.perf_counter() - t0:.1f} s")
        inp, q, k, v = loaded
        o = torch.empty_like(q)
        step, entry, ws_bytes, _ws = make_step(attn, wl, mode, q, k, v, o, stream, dev, args.no_split)
        flops = workload_flops(wl)
        for _ in range(args.sweep_warmup):
            step()
        torch.cuda.synchronize()
        # about args.sweep_seconds of timed launches, at least 10
        probe_ms, _ = time_launches(step, stream, 2)
        steps = int(min(args.steps, max(10, round(args.sweep_seconds * 1e3 / max(probe_ms, 1e-3)))))
        ms_per_step, per = time_launches(step, stream, steps)
        achieved = flops / (per.mean() * 1e-3) / 1e12
        value = flops / (ms_per_step * 1e-3) / 1e12
        log(f"[bench] sweep {name} {mode}: {ms_per_step:.3f} ms/step over {steps} steps -> {value:.1f} TFLOP/s "
            f"({achieved / PEAK_BF16_TFLOPS:.4f} of peak)")
        if args.no_clock or under_profiler():
            clock = {"skipped": "--no-clock" if args.no_clock else "under rocprofv3"}
        else:
            clock = clock_sample(step, float(per.mean()), stream, dev, seconds=args.sweep_clock_seconds)
            clock["sustained_tflops"] = round(flops / (clock["sustained_launch_ms"] * 1e-3) / 1e12, 1)
            clock = {key: clock[key] for key in ("gfx_mhz_mean", "socket_power_w", "mfma_peak_at_clock_tflops",
                                                 "sustained_tflops", "sustained_launch_ms", "under_load",
                                                 "unavailable") if key in clock}
        logical = synth.to_logical(o.view(torch.int16).cpu().numpy().view(np.uint16), wl.layout)
        got = np.stack([logical[b, h, i] for b, h, i in rows])
        res = gate(got, rd[:, ("rtne", "rtna", "rtz").index(mode)], ex)
        log(f"[bench] sweep parity {name} {mode}: {res.summary()}")
        out.append({
            "workload": f"{wl.name}: B={wl.B} H={wl.H} Sq={wl.Sq} Sk={wl.Sk} d=128 {wl.layout.upper()} {mode.upper()}",
            "round_mode": mode, "entry_point": entry, "steps": steps, "warmup": args.sweep_warmup,
            "ms_per_step": round(ms_per_step, 4), "tflops": round(value, 2),
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                         "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic(wl.name),
                         "launch_ms_mean": round(float(per.mean()), 4),
                         "launch_ms_median": round(float(np.median(per)), 4)},
            "clock": clock,
            "parity": {"rows": len(rows), "ok": res.ok, "max_row_ulps": round(res.max_row_ulps, 3),
                       "strict_ulp_hist": res.strict_hist, "rms_excess": round(res.rms_excess, 6)},
        })
        del o, step, _ws
    loaded = None
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding is a "
              "design note, not a measured path", file=sys.stderr)
        sys.exit(2)
    import torch

    import bf16_forward_attention_amd as attn
    from bf16_forward_attention_amd import synth

    if args.workload in synth.VARLEN_WORKLOADS:
        main_varlen(args)
        return
    wl = synth.WORKLOADS[args.workload]
    mode = args.mode or wl.modes[0]
    attn.load_library()
    dev = torch.device("cuda:0")
    log(f"[bench] generating {wl}")
    t0 = time.perf_counter()
    inp = synth.generate(wl)
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s")
    t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = t(inp.q), t(inp.k), t(inp.v)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    masked = wl.mask != "none"
    grouped = wl.kv_heads != wl.H
    step, entry, ws_bytes, ws = make_step(attn, wl, mode, q, k, v, o, stream, dev, args.no_split)
    log(f"[bench] entry point: {entry}")

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t_wall = time.perf_counter()
    ms_per_step, per = time_launches(step, stream, args.steps)
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    flops = workload_flops(wl)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (per.mean() * 1e-3) / 1e12
    log(f"[bench] {ms_per_step:.3f} ms/step (wall {wall_ms / args.steps:.3f}), per-launch mean {per.mean():.3f} "
        f"median {np.median(per):.3f} min {per.min():.3f} ms -> {value:.1f} TFLOP/s")

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calibrate_copy_mib} MiB done")
        del src, dst

    if args.no_clock or under_profiler():
        clock = {"skipped": "--no-clock" if args.no_clock else "under rocprofv3"}
    else:
        clock = clock_sample(step, float(per.mean()), stream, dev)
        clock["sustained_tflops"] = round(flops / (clock["sustained_launch_ms"] * 1e-3) / 1e12, 1)
    log(f"[bench] clock {clock}")
    out_bits = o.view(torch.int16).cpu().numpy().view(np.uint16)
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={wl.B} H={wl.H} Sq={wl.Sq} Sk={wl.Sk} d=128 {wl.layout.upper()} "
                               f"{mode.upper()}" + (f" {wl.mask}" if masked else "")
                               + (f" H_kv={wl.kv_heads}" if grouped else ""),
                   "B": wl.B, "H": wl.H, "H_kv": wl.kv_heads, "Sq": wl.Sq, "Sk": wl.Sk,
                   "head_dim": 128, "layout": wl.layout, "round_mode": mode, "mask": wl.mask,
                   "flops_per_step": flops},
        "entry_point": entry,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(wl.name),
                     "kernel": f"attn_fwd_kernel<{mode.upper()}{', causal' if masked else ''}>"
                               + (" + attn_merge_kernel" if ws_bytes else ""),
                     "launch_ms_mean": round(float(per.mean()), 4),
                     "launch_ms_median": round(float(np.median(per)), 4)},
        "clock": clock,
        "env": run_env(dev),
    }
    if not args.no_cpu_baseline:
        from tests.gate import gate

        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"], rows, ex, rd = cpu_baseline(inp, args.cpu_seconds, args.parity_rows)
        # parity: the timed output on rows the baseline computed
        logical = synth.to_logical(out_bits, wl.layout)
        got = np.stack([logical[b, h, i] for b, h, i in rows])
        res = gate(got, rd[:, ("rtne", "rtna", "rtz").index(mode)], ex)
        result["parity"] = {"rows": len(rows), "ok": res.ok, "max_row_ulps": round(res.max_row_ulps, 3),
                            "strict_ulp_hist": res.strict_hist, "rms_excess": round(res.rms_excess, 6),
                            "rms_floor_violations": res.rms_floor_violations}
        log(f"[bench] parity {res.summary()}")
    # the sweep follows the default workload; under rocprofv3 it is left out unless asked for, so that
    # the traced kernel statistics of the default command hold the headline launches only
    if args.sweep or (args.sweep is None and args.workload == "self8k" and not under_profiler()):
        del q, k, v, o, ws, step
        result["sweep"] = run_sweep(args, dev)
        result["power_reference"] = {"note": POWER_REFERENCE_NOTE, "runs": run_sweep(args, dev, POWER_REFERENCE)}
    print(json.dumps(result), flush=True)


def varlen_visible_pairs(wl) -> np.ndarray:
    """Visible (query, key) pairs of each sequence of a variable-length workload."""
    out = []
    for Sq, Sk in zip(wl.lengths_q, wl.lengths_k):
        i = np.arange(Sq, dtype=np.int64)
        if wl.mask == "none":
            out.append(Sq * Sk)
        else:
            off = 0 if wl.mask == "causal" else Sk - Sq
            out.append(int(np.clip(i + off + 1, 0, Sk).sum()))
    return np.array(out, dtype=np.int64)


def main_varlen(args):
    """The same protocol for a packed variable-length batch (attn_fwd_bf16_varlen)."""
    import torch

    import bf16_forward_attention_amd as attn
    from bf16_forward_attention_amd import synth

    wl = synth.VARLEN_WORKLOADS[args.workload]
    mode = args.mode or wl.modes[0]
    attn.load_library()
    dev = torch.device("cuda:0")
    log(f"[bench] generating {wl.name}: {wl.B} sequences, {sum(wl.lengths_q)} query / {sum(wl.lengths_k)} key rows")
    inp = synth.generate_varlen(wl)
    t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = t(inp.q), t(inp.k), t(inp.v)
    cq, ck = torch.from_numpy(inp.cu_q).to(dev), torch.from_numpy(inp.cu_k).to(dev)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    max_q = max(wl.lengths_q)
    entry = f"attn_fwd_bf16_varlen(B={wl.B}, H_kv={wl.H_kv}, {wl.mask})"
    log(f"[bench] entry point: {entry}")

    def step():
        st = attn.attn_fwd_bf16_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), 0, cq.data_ptr(),
                                       ck.data_ptr(), wl.B, wl.H, wl.H_kv, q.shape[0], k.shape[0], max_q,
                                       attn.ROUND_MODES[mode], attn.MASKS[wl.mask], stream.cuda_stream)
        if st != 0:
            raise attn.AttnError(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    ms_per_step = starts[0].elapsed_time(ends[-1]) / args.steps
    flops = 4.0 * 128 * wl.H * float(varlen_visible_pairs(wl).sum())
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (per.mean() * 1e-3) / 1e12
    log(f"[bench] {ms_per_step:.3f} ms/step, per-launch mean {per.mean():.3f} median {np.median(per):.3f} ms "
        f"-> {value:.1f} TFLOP/s")
    if args.no_clock or under_profiler():
        clock = {"skipped": "--no-clock" if args.no_clock else "under rocprofv3"}
    else:
        clock = clock_sample(step, float(per.mean()), stream, dev)
        clock["sustained_tflops"] = round(flops / (clock["sustained_launch_ms"] * 1e-3) / 1e12, 1)
    log(f"[bench] clock {clock}")
    out_bits = o.view(torch.int16).cpu().numpy().view(np.uint16)
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.B} packed sequences of {min(wl.lengths_q)}..{max(wl.lengths_q)} "
                               f"tokens ({sum(wl.lengths_q)} in all), H={wl.H} H_kv={wl.H_kv} d=128 "
                               f"{mode.upper()} {wl.mask}",
                   "lengths_q": list(wl.lengths_q), "lengths_k": list(wl.lengths_k), "H": wl.H, "H_kv": wl.H_kv,
                   "head_dim": 128, "round_mode": mode, "mask": wl.mask, "flops_per_step": flops},
        "entry_point": entry,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(wl.name),
                     "kernel": f"attn_fwd_kernel<{mode.upper()}, varlen{', causal' if wl.mask != 'none' else ''}>",
                     "launch_ms_mean": round(float(per.mean()), 4),
                     "launch_ms_median": round(float(np.median(per)), 4)},
        "clock": clock,
        "env": run_env(dev),
    }
    if not args.no_cpu_baseline:
        import oracle
        from tests.gate import gate

        # CPU baseline: the oracle on every query row of one head per sequence (head b mod H),
        # sequence after sequence until about --cpu-seconds; the parity check then compares the
        # timed output with rows of that sample (the oracle runs only here)
        threads = oracle.default_threads()
        sample, pairs, t0 = [], 0, time.perf_counter()
        seq_pairs = varlen_visible_pairs(wl)
        budget = args.cpu_seconds
        done = []
        for b in range(wl.B):
            rows_b = [(int(tq), b % wl.H) for tq in range(inp.cu_q[b], inp.cu_q[b + 1])]
            ex_b, rd_b = oracle.attn_rows_varlen(inp.q, inp.k, inp.v, inp.cu_q, inp.cu_k, rows_b, wl.mask, threads)
            done.append((rows_b, ex_b, rd_b))
            sample.append(b)
            pairs += int(seq_pairs[b])
            if time.perf_counter() - t0 > budget:
                break
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": 4.0 * 128 * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"every query row of one head (b mod {wl.H}) of sequences {sample[0]}.."
                                            f"{sample[-1]} of {wl.name} ({pairs} visible pairs, fp64 with 3 "
                                            f"roundings), {dt:.2f} s"}
        rows = [r for rb, _, _ in done for r in rb]
        ex = np.concatenate([e for _, e, _ in done])
        rd = np.concatenate([r_ for _, _, r_ in done])
        idx = np.unique(np.linspace(0, len(rows) - 1, min(args.parity_rows, len(rows))).astype(np.int64))
        got = np.stack([out_bits[rows[i][0], rows[i][1]] for i in idx])
        res = gate(got, rd[idx, ("rtne", "rtna", "rtz").index(mode)], ex[idx])
        result["parity"] = {"rows": len(idx), "ok": res.ok, "max_row_ulps": round(res.max_row_ulps, 3),
                            "strict_ulp_hist": res.strict_hist}
        log(f"[bench] parity {res.summary()}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
