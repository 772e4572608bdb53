#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill|decode|prefill_fp8|rolling|softmax]
                    [--no-cpu-baseline] [--no-decode]
    python bench.py --summarize-profiles DIR   (host only: rocprofv3 CSVs -> profiles/)

A step is one forward pass over one batch of synthetic input:

* prefill (default): ``fa_fwd`` on the causal bf16 prefill workload
  (B=4, H=32, 4096 x 4096, d=128) -- the headline TFLOP/s figure;
* decode (also measured in the same run unless ``--no-decode``):
  ``fa_fwd_splitkv`` + ``fa_combine`` on the split-KV decode workload
  (B=16, H=32, Hkv=8, Nk=32768, d=128, 16 splits), in GB/s;
* rolling (same condition): streaming decode over a rolling KV cache with
  attention sinks -- ``fa_kv_append`` of one token + ``fa_decode_rolling``
  + ``fa_combine`` (B=16, H=32, Hkv=8, d=128, window 4096, 4 sinks, 4
  splits, position 65535), in GB/s;
* softmax (same condition): ``fa_softmax`` (online normaliser) and
  ``fa_softmax_topk`` (k = 8) on 512 rows of 256000 fp32 logits, in GB/s;
``--workload rolling`` and ``--workload softmax`` run only that leg and print
its object (for profiling those kernels in runs of their own).

* prefill_fp8 (same condition; ``--workload prefill_fp8`` runs it alone):
  ``fa_fwd_fp8`` on the causal prefill shape with E4M3 Q, K, V, in TFLOP/s
  against the 5 PFLOP/s dense fp8 peak.

Inputs are seeded synthetic tensors (online_softmax_tiled_amd.workloads),
resident in HBM before timing starts.  Kernel durations are taken with HIP
events recorded on the stream the kernels are launched on (torch's current
stream).  Prints ONE JSON line.  ``cpu_baseline`` times the fp64 CPU oracle
on a bounded row sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from online_softmax_tiled_amd import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# Untimed wall time each leg runs before its counted warm-up launches: an
# idle MI355X takes tens of milliseconds to reach its working clocks, and a
# few warm-up launches of a sub-millisecond kernel do not cover that.
SETTLE_MS = 200.0
METRIC = "attention fwd TFLOP/s (% bf16 MFMA peak); decode GB/s (% HBM peak)"
PREFILL = "bf16_causal_b4_h32_n4096_d128"
DECODE = "bf16_splitkv_decode_b16_h32kv8_nk32768_d128"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "prefill": ["online_softmax_tiled_amd/csrc/fa_fwd_bf16_wide.hip", "online_softmax_tiled_amd/csrc/fa_bf16_tile.h",
                "online_softmax_tiled_amd/csrc/fa_tile.h", "online_softmax_tiled_amd/csrc/fa_device.h"],
    "decode": ["online_softmax_tiled_amd/csrc/fa_splitkv.hip", "online_softmax_tiled_amd/csrc/fa_device.h"],
    "prefill_fp8": ["online_softmax_tiled_amd/csrc/fa_fwd_fp8.hip", "online_softmax_tiled_amd/csrc/fa_tile.h",
                    "online_softmax_tiled_amd/csrc/fa_device.h"],
    "rolling_decode": ["online_softmax_tiled_amd/csrc/fa_splitkv.hip", "online_softmax_tiled_amd/csrc/fa_device.h"],
    "softmax": ["online_softmax_tiled_amd/csrc/fa_softmax.hip"],
    "topk": ["online_softmax_tiled_amd/csrc/fa_softmax.hip"],
}


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kind: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    or None when absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kind)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(kind):
        return None
    return rec.get("bytes_per_launch")


# Other prefill configurations reported beside the headline one (TFLOP/s and
# fraction of the bf16 peak): non-causal small heads, and causal GQA with
# sliding windows on even heads and a soft-cap (the fixed-maximum kernel).
OTHER_PREFILL = ("bf16_b1_h8_n1024_d64", "bf16_gqa_swa_softcap_h32kv8_n16384_d128")


def to_device(inp, torch):
    return {n: torch.from_numpy(inp[n]).to(torch.bfloat16).cuda() for n in "qkv"}


class Timing:
    """Event timings of one leg: `total_ms` between one event pair around
    all K steps, and per step (and per kernel of a step) the time between
    events recorded before and after it on the launch stream."""

    def __init__(self, total_ms, wall_s, step_ms, part_ms):
        self.total_ms, self.wall_s = total_ms, wall_s
        self.step_ms, self.part_ms = step_ms, part_ms

    @staticmethod
    def stats(ms):
        a = np.asarray(ms, dtype=np.float64)
        return {"mean_ms": round(float(a.mean()), 5), "median_ms": round(float(np.median(a)), 5),
                "min_ms": round(float(a.min()), 5), "max_ms": round(float(a.max()), 5)}

    def per_step(self, steps):
        return self.total_ms / steps


def time_leg(parts, steps, warmup, settle_ms, torch):
    """One leg: a step launches every callable in `parts` in order.  Runs
    untimed launches for `settle_ms` of wall time (the GPU leaves its idle
    clock state; 0 skips this) and `warmup` untimed steps; then the timed
    region: exactly `steps` steps back to back between one pair of events
    (total_ms: value and ms_per_step).  A second pass of `steps` steps then
    records events before and after every kernel of every step, for the
    per-launch durations (mean, median, minimum) of each kernel; those
    events would add their own few microseconds to the first pass.  All
    events are recorded on the launch stream."""
    def step():
        for p in parts:
            p()
    if settle_ms > 0:
        t_end = time.perf_counter() + settle_ms * 1e-3
        while time.perf_counter() < t_end:
            for _ in range(4):
                step()
            torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total = start.elapsed_time(end)
    n = len(parts)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    for i in range(steps):
        e = ev[i]
        e[0].record()
        for j, p in enumerate(parts):
            p()
            e[j + 1].record()
    torch.cuda.synchronize()
    step_ms = [e[0].elapsed_time(e[n]) for e in ev]
    part_ms = [[e[j].elapsed_time(e[j + 1]) for e in ev] for j in range(n)]
    return Timing(total, wall, step_ms, part_ms)


# ---------------------------------------------------------------- the legs
# Each prepare_* function generates the leg's seeded inputs, uploads them and
# returns the callables of one step; every leg is prepared before any leg is
# timed, so the GPU never waits for host-side input generation between legs.

def prepare_prefill(torch, fa, name=PREFILL):
    w = wl.WORKLOADS[name]
    t = to_device(wl.generate(w), torch)
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    hw = list(w.head_window) if w.head_window else None
    # The argument block is built once (the smaller workloads' launches take
    # tens of microseconds; rebuilding it per launch would time the host).
    import ctypes
    from online_softmax_tiled_amd.fa import FwdArgs
    hw_arr = (ctypes.c_int32 * len(hw))(*hw) if hw else None
    a = FwdArgs(0, t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(), lse.data_ptr(),
                w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, float(w.scale), int(w.causal), int(w.window),
                float(w.softcap), ctypes.cast(hw_arr, ctypes.POINTER(ctypes.c_int32)) if hw else None,
                torch.cuda.current_stream().cuda_stream or None)
    lib, ref = fa.load_library(), ctypes.byref(a)
    keep = (t, o, lse, hw_arr, a)

    def launch():
        if lib.fa_fwd_ex(ref) != 0:
            raise RuntimeError("fa_fwd_ex failed")
    launch.keep = keep
    return w, [launch]


def prepare_prefill_fp8(torch, fa):
    w = wl.FP8_PREFILL
    x = wl.generate_fp8(w)
    t = {n: torch.from_numpy(x[n]).cuda() for n in "qkv"}
    o = torch.empty((w.B, w.H, w.Nq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    args = (t["q"], t["k"], t["v"], o, lse, w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, w.scale, x["q_descale"],
            x["k_descale"], x["v_descale"], int(w.causal), w.window)

    def launch():
        fa.fa_fwd_fp8(*args)
    return w, [launch]


def prepare_decode(torch, fa):
    w = wl.WORKLOADS[DECODE]
    t = to_device(wl.generate(w), torch)
    S = w.num_splits
    o_part = torch.empty((w.B, w.H, w.Nq, S, w.d), dtype=torch.float32, device="cuda")
    m_part = torch.empty((w.B, w.H, w.Nq, S), dtype=torch.float32, device="cuda")
    l_part = torch.empty_like(m_part)
    o = torch.empty((w.B, w.H, w.Nq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")

    def split():
        fa.fa_fwd_splitkv(t["q"], t["k"], t["v"], o_part, m_part, l_part, w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d,
                          w.scale, int(w.causal), w.window, w.softcap, S)

    def combine():
        fa.fa_combine(o_part, m_part, l_part, o, lse, w.B, w.H, w.Nq, w.d, S, 0)
    return w, [split, combine]


def prepare_rolling(torch, fa):
    """Streaming decode over a rolling KV cache with attention sinks: a step
    appends one token's K/V (fa_kv_append) and runs fa_decode_rolling +
    fa_combine for its query, at a fixed position far into the stream."""
    w = wl.ROLLING
    rng = np.random.default_rng(w.seed)

    def rand(*shape):
        return torch.from_numpy(wl.round_bf16(rng.standard_normal(shape).astype(np.float32))) \
            .to(torch.bfloat16).cuda()

    rows = w.sinks + w.window
    kc, vc = rand(w.B, w.Hkv, rows, w.d), rand(w.B, w.Hkv, rows, w.d)
    kn, vn = rand(w.B, w.Hkv, 1, w.d), rand(w.B, w.Hkv, 1, w.d)
    q = rand(w.B, w.H, 1, w.d)
    S = w.num_splits
    o_part = torch.empty((w.B, w.H, 1, S, w.d), dtype=torch.float32, device="cuda")
    m_part = torch.empty((w.B, w.H, 1, S), dtype=torch.float32, device="cuda")
    l_part = torch.empty_like(m_part)
    o = torch.empty((w.B, w.H, 1, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, 1), dtype=torch.float32, device="cuda")

    def append():
        fa.fa_kv_append(kn, vn, kc, vc, w.B, w.Hkv, 1, w.d, w.pos, w.window, w.sinks)

    def decode():
        fa.fa_decode_rolling(q, kc, vc, o_part, m_part, l_part, w.B, w.H, w.Hkv, w.d, w.pos, w.window, w.sinks,
                             w.scale, 0.0, S)

    def combine():
        fa.fa_combine(o_part, m_part, l_part, o, lse, w.B, w.H, 1, w.d, S, 0)
    return w, [append, decode, combine]


def prepare_softmax(torch, fa):
    """Row softmax with the online normaliser and the fused softmax top-k on
    vocabulary-sized rows (fp32); torch's softmax and softmax + topk on the
    same rows are timed beside them for context."""
    w = wl.SOFTMAX
    rng = np.random.default_rng(w.seed)
    x = torch.from_numpy((rng.standard_normal((w.rows, w.n)) * 3.0).astype(np.float32)).cuda()
    y = torch.empty_like(x)
    probs = torch.empty((w.rows, w.k), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.rows, w.k), dtype=torch.int32, device="cuda")

    def sm():
        fa.fa_softmax(x, y, None, w.rows, w.n, fa.fa.FA_DTYPE_FP32)

    def tk():
        fa.fa_softmax_topk(x, probs, idx, None, w.rows, w.n, w.k, fa.fa.FA_DTYPE_FP32)

    def torch_sm():
        torch.softmax(x, dim=-1)

    def torch_tk():
        torch.topk(torch.softmax(x, dim=-1), w.k, dim=-1)
    return w, {"softmax": [sm], "topk": [tk], "torch_softmax": [torch_sm], "torch_softmax_topk": [torch_tk]}


def prepare_standard_attention(torch):
    """Standard attention with the score matrix materialised in HBM (two
    torch bf16 matrix products and an fp32 softmax over the masked scores),
    on the first batch element of the causal prefill workload: the baseline
    that the pages' FlashAttention speedup figure compares against."""
    w = wl.WORKLOADS[PREFILL].with_(B=1)
    t = to_device(wl.generate(w), torch)
    q, v = t["q"], t["v"]
    kt = t["k"].transpose(-1, -2).contiguous()
    mask = torch.ones((w.Nq, w.Nk), dtype=torch.bool, device="cuda").triu_(1)

    def launch():
        s = torch.matmul(q, kt).float().mul_(w.scale).masked_fill_(mask, float("-inf"))
        p = torch.softmax(s, dim=-1).to(torch.bfloat16)
        del s
        torch.matmul(p, v)
    return w, [launch]


def cpu_baseline(w, target_s: float = 15.0, max_threads: int = 16):
    """Time the fp64 oracle on a strided row sample of workload ``w``."""
    import oracle
    if w.dtype == "fp8":
        from oracle import fp8 as ofp8
        x = wl.generate_fp8(w)
        q, k, v = (ofp8.dequantise(x[n], x[n + "_descale"]) for n in "qkv")
    else:
        inp = wl.generate(w)
        q, k, v = (inp[n].astype(np.float64) for n in "qkv")
    total = w.B * w.H * w.Nq
    threads = max(1, min(max_threads, len(os.sched_getaffinity(0))))
    hw = list(w.head_window) if w.head_window else None
    counts = np.broadcast_to(wl.visible_counts(w)[None], (w.B, w.H, w.Nq)).reshape(-1)

    def run(rows):
        t0 = time.perf_counter()
        oracle.attention(q, k, v, w.scale, causal=w.causal, window=w.window, head_window=hw,
                         softcap=w.softcap, rows=rows, nthreads=threads)
        return time.perf_counter() - t0

    stride = max(1, total // 2048)
    pilot = np.arange(0, total, stride, dtype=np.int64)
    tp = run(pilot)
    stride = max(1, int(stride * tp / target_s))
    rows = np.arange(0, total, stride, dtype=np.int64)
    secs = run(rows)
    flops = 4 * w.d * int(counts[rows].sum())
    if w.num_splits:
        value, unit = wl.algorithmic_bytes(w) * len(rows) / total / secs / 1e9, "GB/s"
    else:
        value, unit = flops / secs / 1e12, "TFLOP/s"
    what = (f"all {total} query rows" if stride == 1 else
            f"one query row in {stride} ({len(rows)} of {total})")
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{what} of {w.name} ({flops / 1e9:.1f} GFLOP fp64 in {secs:.1f} s)",
            "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def device_info(torch):
    """The GPU's compute-unit count and maximum clock as rocminfo reports
    them, the dense bf16 MFMA peak they imply (4 SIMDs per CU, each 1024
    bf16 FLOP per clock on gfx950), and a measured device-to-device copy
    rate as a check of the HBM figure."""
    import subprocess
    info = {"name": torch.cuda.get_device_name(0),
            "torch_multiprocessor_count": torch.cuda.get_device_properties(0).multi_processor_count}
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
        agent = None
        for blk in out.split("Agent ")[1:]:
            if "gfx950" in blk and "Compute Unit:" in blk:
                agent = blk
                break
        if agent is not None:
            def field(key):
                for line in agent.splitlines():
                    if line.strip().startswith(key):
                        return line.split(":", 1)[1].split()[0]
                return None
            cu, mhz = int(field("Compute Unit")), int(field("Max Clock Freq. (MHz)"))
            info["rocminfo"] = {"compute_units": cu, "max_clock_mhz": mhz,
                                "bf16_dense_peak_tflops": round(cu * 4 * 1024 * mhz * 1e6 / 1e12, 1),
                                "fp8_dense_peak_tflops": round(cu * 4 * 2048 * mhz * 1e6 / 1e12, 1)}
    except (OSError, subprocess.SubprocessError, ValueError, TypeError):
        info["rocminfo"] = None
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_()
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    times = []
    for _ in range(10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    info["copy_1GiB"] = {"median_ms": round(float(np.median(times)), 4),
                         "gbs_read_plus_write": round(2 * n / (float(np.median(times)) * 1e-3) / 1e9, 1)}
    del src, dst
    return info


# The pages' own figures (context, not targets: none is an MI355X number).
PAGES_CONTEXT = [
    {"figure": "FlashAttention speedup over standard attention, often quoted as 3x to 5x",
     "source": "Transformers & Math, Module 16, section 16.2 (hardware not stated)",
     "measured_here": "standard_attention.speedup (same GPU, first batch element of the causal prefill workload)"},
    {"figure": "online-normaliser softmax up to 1.3x faster than the safe softmax",
     "source": "Online normalizer calculation for softmax, abstract (hardware not stated)",
     "measured_here": "softmax.softmax.byte_ratio_vs_three_pass, softmax.softmax.speedup_vs_torch"},
    {"figure": "softmax fused with top-k up to 5x faster",
     "source": "Online normalizer calculation for softmax, abstract (hardware not stated)",
     "measured_here": "softmax.topk.byte_ratio_vs_unfused, softmax.topk.speedup_vs_torch"},
    {"figure": "block-wise CPU attention 2-5x faster, about 75% less memory",
     "source": "oxios_kernel flash_attention.rs, module documentation (single-thread CPU, f32)",
     "measured_here": "cpu_baseline (the oracle is the direct definition, not a blocked CPU kernel)"},
]


# rocprofv3 runs whose output --summarize-profiles reads (DIR = their -d root).
# The prefill and decode kernels are profiled in runs of their own legs
# (the rolling-cache leg launches the same decode kernel at another shape).
PROFILE_RUNS = {
    "trace_prefill": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace_prefill -o run -- "
                     "python bench.py --no-cpu-baseline --no-decode",
    "trace_decode": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace_decode -o run -- "
                    "python bench.py --no-cpu-baseline --workload decode",
    "FETCH_SIZE_prefill": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/FETCH_SIZE_prefill -o run -- "
                          "python bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-decode",
    "WRITE_SIZE_prefill": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/WRITE_SIZE_prefill -o run -- "
                          "python bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-decode",
    "FETCH_SIZE_decode": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/FETCH_SIZE_decode -o run -- "
                         "python bench.py --steps 3 --warmup 1 --no-cpu-baseline --workload decode",
    "WRITE_SIZE_decode": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/WRITE_SIZE_decode -o run -- "
                         "python bench.py --steps 3 --warmup 1 --no-cpu-baseline --workload decode",
    "trace_prefill_fp8": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace_prefill_fp8 -o run -- "
                         "python bench.py --no-cpu-baseline --workload prefill_fp8",
    "FETCH_SIZE_prefill_fp8": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/FETCH_SIZE_prefill_fp8 -o run "
                              "-- python bench.py --steps 3 --warmup 1 --no-cpu-baseline --workload prefill_fp8",
    "WRITE_SIZE_prefill_fp8": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/WRITE_SIZE_prefill_fp8 -o run "
                              "-- python bench.py --steps 3 --warmup 1 --no-cpu-baseline --workload prefill_fp8",
    "trace_rolling": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace_rolling -o run -- "
                     "python bench.py --no-cpu-baseline --workload rolling",
    "trace_softmax": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace_softmax -o run -- "
                     "python bench.py --no-cpu-baseline --workload softmax",
    "FETCH_SIZE_rolling": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/FETCH_SIZE_rolling -o run -- "
                          "python bench.py --steps 3 --warmup 1 --no-cpu-baseline --workload rolling",
    "WRITE_SIZE_rolling": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/WRITE_SIZE_rolling -o run -- "
                          "python bench.py --steps 3 --warmup 1 --no-cpu-baseline --workload rolling",
    "FETCH_SIZE_softmax": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/FETCH_SIZE_softmax -o run -- "
                          "python bench.py --steps 3 --warmup 1 --no-cpu-baseline --workload softmax",
    "WRITE_SIZE_softmax": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/WRITE_SIZE_softmax -o run -- "
                          "python bench.py --steps 3 --warmup 1 --no-cpu-baseline --workload softmax",
    "copy_FETCH_SIZE": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/copy_FETCH_SIZE -o run -- "
                       "python bench.py --copy-calibration",
    "copy_WRITE_SIZE": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/copy_WRITE_SIZE -o run -- "
                       "python bench.py --copy-calibration",
}
KERNELS = {"prefill": "fwd_bf16_wide_kernel<1, false, false, false>", "decode": "splitkv_decode_kernel<128, 4, false>",
           "combine": "combine_few_kernel<128, 16>", "prefill_fp8": "fwd_fp8_kernel<128>",
           "rolling_decode": "splitkv_decode_kernel<128, 4, false>", "kv_append": "kv_append_kernel<128>",
           "softmax": "softmax_kernel<false, 4>", "topk": "softmax_topk_kernel<false, 4>",
           "copy": "__amd_rocclr_copyBuffer"}


def _csv(path):
    import csv
    import glob
    files = glob.glob(path)
    if not files:
        raise SystemExit(f"no file matches {path}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _counter_kib(d, run, kernel):
    """Mean over dispatches of one counter (KiB per dispatch) for `kernel`."""
    per = {}
    for r in _csv(os.path.join(d, run, "*counter_collection.csv")):
        if kernel in r["Kernel_Name"]:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"{run}: no dispatch of {kernel}")
    return sum(per.values()) / len(per)


def summarize_profiles(d):
    """Write profiles/hbm_traffic.json and the two kernel-trace summaries
    from the rocprofv3 output under d (the runs in PROFILE_RUNS)."""
    cmds = {k: v.format(d=d) for k, v in PROFILE_RUNS.items()}
    leg = {"prefill": "prefill", "decode": "decode", "combine": "decode", "prefill_fp8": "prefill_fp8",
           "rolling_decode": "rolling", "softmax": "softmax", "topk": "softmax"}

    def stat(kernel, run):
        stats = {r["Name"]: r for r in _csv(os.path.join(d, run, "*kernel_stats.csv"))}
        for name, r in stats.items():
            if kernel in name:
                return name.replace("void fa::(anonymous namespace)::", ""), int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, \
                    float(r["MaxNs"]) / 1e3
        raise SystemExit(f"trace: no kernel {kernel}")

    copy_bytes = 1 << 30
    cf = _counter_kib(d, "copy_FETCH_SIZE", KERNELS["copy"])
    cw = _counter_kib(d, "copy_WRITE_SIZE", KERNELS["copy"])
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    traffic = {
        "note": "HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch, "
                "mean over dispatches), each scaled by what the same counter reads for a 1 GiB device copy "
                "(__amd_rocclr_copyBuffer).  bench.py reports these only while source_hash matches the "
                "kernel sources.  Written by: python bench.py --summarize-profiles DIR.",
        "commands": [cmds[k] for k in ("FETCH_SIZE_prefill", "WRITE_SIZE_prefill", "FETCH_SIZE_decode",
                                       "WRITE_SIZE_decode", "FETCH_SIZE_prefill_fp8", "WRITE_SIZE_prefill_fp8",
                                       "FETCH_SIZE_rolling", "WRITE_SIZE_rolling", "FETCH_SIZE_softmax",
                                       "WRITE_SIZE_softmax", "copy_FETCH_SIZE", "copy_WRITE_SIZE")],
        "copy_calibration": {"bytes": copy_bytes, "fetch_kib": round(cf, 1), "write_kib": round(cw, 1)},
    }
    hbm = {}
    for kind in ("prefill", "decode", "combine", "prefill_fp8", "rolling_decode", "softmax", "topk"):
        f = _counter_kib(d, "FETCH_SIZE_" + leg[kind], KERNELS[kind])
        w_ = _counter_kib(d, "WRITE_SIZE_" + leg[kind], KERNELS[kind])
        rb, wb = f * 1024 * fs, w_ * 1024 * ws
        hbm[kind] = (rb, wb)
        rec = {"kernel": KERNELS[kind], "fetch_kib_per_dispatch": round(f, 1),
               "write_kib_per_dispatch": round(w_, 1), "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
               "bytes_per_launch": int(round(rb + wb))}
        if kind in KERNEL_SOURCES:
            rec["source_hash"] = source_hash(kind)
        traffic[kind] = rec
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")

    wp, wd = wl.WORKLOADS[PREFILL], wl.WORKLOADS[DECODE]
    name, calls, avg, mn, mx = stat(KERNELS["prefill"], "trace_prefill")
    flops = wl.algorithmic_flops(wp)
    rb, wb = hbm["prefill"]
    qkv_bytes = 2 * (wp.B * wp.H * wp.Nq * wp.d + 2 * wp.B * wp.Hkv * wp.Nk * wp.d)
    md = f"""# fwd_bf16_wide_kernel on the causal prefill workload (B=4, H=32, Nq=Nk=4096, d=128, bf16)

Command (run from the repository root on one MI355X):

    {cmds["trace_prefill"]}

Kernel trace statistics (`run_kernel_stats.csv`; every dispatch of the run,
the bench's warm-up launches included):

| kernel | calls | average (us) | min (us) | max (us) |
|---|---|---|---|---|
| {name[:90]} | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} |

Algorithmic work per launch: {flops:,} FLOP (4*d per visible query-key pair,
N(N+1)/2 pairs per head).  At the trace's average duration this is
{flops / (avg * 1e-6) / 1e12:.0f} TFLOP/s ({flops / (avg * 1e-6) / 1e12 / PEAK_BF16_TFLOPS * 100:.1f}% of the 2.5 PFLOP/s dense bf16 peak);
at the minimum, {flops / (mn * 1e-6) / 1e12:.0f} TFLOP/s.

HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE,
scaled by a 1 GiB copy; see hbm_traffic.json for the commands): read {rb / 1e6:.1f} MB,
written {wb / 1e6:.1f} MB, total {(rb + wb) / 1e6:.1f} MB, against {wl.algorithmic_bytes(wp) / 1e6:.1f} MB of
algorithmic bytes (Q, K, V read once, O and lse written once).  Reads are
{rb / qkv_bytes:.2f}x the {qkv_bytes / 1e6:.1f} MB of Q, K and V: most re-reads of a head's K and V by
its {(wp.Nq + 255) // 256} query tiles hit in L2 / MALL, because each XCD works on a few heads at a
time (blocks ordered longest tile first within clusters of heads).
"""
    with open(os.path.join(ROOT, "profiles", f"fwd_bf16_causal_b4_h32_n4096_d128.md"), "w") as f:
        f.write(md)

    name, calls, avg, mn, mx = stat(KERNELS["decode"], "trace_decode")
    cname, ccalls, cavg, cmn, cmx = stat(KERNELS["combine"], "trace_decode")
    S = wd.num_splits
    part_bytes = wd.B * wd.H * wd.Nq * S * (wd.d + 2) * 4
    split_bytes = wl.algorithmic_bytes(wd) - part_bytes - (wd.B * wd.H * wd.Nq * (wd.d * 2 + 4))
    rb, wb = hbm["decode"]
    crb, cwb = hbm["combine"]
    md = f"""# splitkv_decode_kernel + combine_few_kernel on the split-KV decode workload (B=16, H=32, Hkv=8, Nq=1, Nk=32768, d=128, 16 splits, bf16)

Command (run from the repository root on one MI355X):

    {cmds["trace_decode"]}

Kernel trace statistics (`run_kernel_stats.csv`; the bench runs the split
kernel both inside split+combine steps and alone, warm-up included):

| kernel | calls | average (us) | min (us) | max (us) |
|---|---|---|---|---|
| {name[:90]} | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} |
| {cname[:90]} | {ccalls} | {cavg:.1f} | {cmn:.1f} | {cmx:.1f} |

Algorithmic bytes of the split kernel per launch: {split_bytes:,} (K and V
read once per K/V head, Q read, fp32 partials written).  At the trace's
average duration: {split_bytes / (avg * 1e-6) / 1e9:.0f} GB/s ({split_bytes / (avg * 1e-6) / 1e9 / PEAK_HBM_GBS * 100:.1f}% of the 8 TB/s HBM3E peak).
Split + combine: {avg + cavg:.1f} us for {wl.algorithmic_bytes(wd):,} algorithmic bytes,
{wl.algorithmic_bytes(wd) / ((avg + cavg) * 1e-6) / 1e9:.0f} GB/s ({wl.algorithmic_bytes(wd) / ((avg + cavg) * 1e-6) / 1e9 / PEAK_HBM_GBS * 100:.1f}%).

HBM traffic per launch (FETCH_SIZE / WRITE_SIZE scaled by a 1 GiB copy; see
hbm_traffic.json): split kernel read {rb / 1e9:.3f} GB, written {wb / 1e6:.2f} MB
(algorithmic {split_bytes / 1e9:.3f} GB); combine {(crb + cwb) / 1e6:.2f} MB
(algorithmic {part_bytes / 1e6:.2f} MB of partials read + {wd.B * wd.H * wd.Nq * (wd.d * 2 + 4) / 1e6:.2f} MB of O and lse written).
"""
    with open(os.path.join(ROOT, "profiles", f"splitkv_decode_b16_h32kv8_nk32768_d128.md"), "w") as f:
        f.write(md)
    w8 = wl.FP8_PREFILL
    name, calls, avg, mn, mx = stat(KERNELS["prefill_fp8"], "trace_prefill_fp8")
    flops = wl.algorithmic_flops(w8)
    rb, wb = hbm["prefill_fp8"]
    md = f"""# fwd_fp8_kernel on the causal prefill shape with E4M3 inputs (B=4, H=32, Nq=Nk=4096, d=128)

Command (run from the repository root on one MI355X):

    {cmds["trace_prefill_fp8"]}

Kernel trace statistics (`run_kernel_stats.csv`; every dispatch of the run,
warm-up included):

| kernel | calls | average (us) | min (us) | max (us) |
|---|---|---|---|---|
| {name[:90]} | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} |

Algorithmic work per launch: {flops:,} FLOP.  At the trace's average duration
this is {flops / (avg * 1e-6) / 1e12:.0f} TFLOP/s ({flops / (avg * 1e-6) / 1e12 / PEAK_FP8_TFLOPS * 100:.1f}% of the 5 PFLOP/s dense fp8 peak,
{flops / (avg * 1e-6) / 1e12 / PEAK_BF16_TFLOPS * 100:.1f}% of the bf16 one).

HBM traffic per launch (FETCH_SIZE / WRITE_SIZE scaled by a 1 GiB copy):
read {rb / 1e6:.1f} MB, written {wb / 1e6:.1f} MB, against {wl.algorithmic_bytes(w8) / 1e6:.1f} MB of algorithmic
bytes (one-byte Q, K, V read once, bf16 O and fp32 lse written once).
"""
    with open(os.path.join(ROOT, "profiles", "fwd_fp8_causal_b4_h32_n4096_d128.md"), "w") as f:
        f.write(md)
    wr = wl.ROLLING
    rows = []
    for kind in ("kv_append", "rolling_decode", "combine"):
        rows.append(stat(KERNELS[kind], "trace_rolling"))
    dec_bytes = (2 * wr.rows * wr.B * wr.Hkv * wr.d * 2 + wr.B * wr.H * wr.d * 2
                 + wr.B * wr.H * wr.num_splits * (wr.d + 2) * 4)
    davg = rows[1][2]
    rb, wb = hbm["rolling_decode"]
    table = "\n".join(f"| {n[:90]} | {c} | {a:.1f} | {mn_:.1f} | {mx_:.1f} |" for n, c, a, mn_, mx_ in rows)
    md = f"""# Streaming decode over a rolling KV cache with attention sinks (B=16, H=32, Hkv=8, d=128, window 4096, 4 sinks, position 65535, 4 splits, bf16)

Command (run from the repository root on one MI355X):

    {cmds["trace_rolling"]}

Kernel trace statistics (`run_kernel_stats.csv`; one step = append + decode
+ combine, and the decode kernel also alone; warm-up included):

| kernel | calls | average (us) | min (us) | max (us) |
|---|---|---|---|---|
{table}

Decode kernel: {dec_bytes:,} algorithmic bytes per launch (the {wr.rows} filled
cache rows of K and V per (batch, K/V head) read once, Q read, fp32 partials
written); at the trace's average duration {dec_bytes / (davg * 1e-6) / 1e9:.0f} GB/s
({dec_bytes / (davg * 1e-6) / 1e9 / PEAK_HBM_GBS * 100:.1f}% of 8 TB/s).  HBM traffic per decode launch (FETCH_SIZE /
WRITE_SIZE scaled by a 1 GiB copy): read {rb / 1e6:.1f} MB, written {wb / 1e6:.1f} MB.
"""
    with open(os.path.join(ROOT, "profiles", "rolling_decode_b16_h32kv8_w4096_s4_d128.md"), "w") as f:
        f.write(md)

    ws_ = wl.SOFTMAX
    sb = wl.softmax_bytes(ws_)
    lines = []
    for kind, nb, what in (("softmax", sb["softmax_online"], "two reads of x, one write of y"),
                           ("topk", sb["topk_fused"], "one read of x, k pairs written")):
        name, calls, avg, mn, mx = stat(KERNELS[kind], "trace_softmax")
        rb, wb = hbm[kind]
        lines.append((name, calls, avg, mn, mx, nb, what, rb, wb))
    table = "\n".join(f"| {n[:60]} | {c} | {a:.1f} | {mn_:.1f} | {mx_:.1f} |" for n, c, a, mn_, mx_, *_ in lines)
    detail = "\n".join(
        f"* {n.split('(')[0]}: {nb:,} algorithmic bytes ({what}); {nb / (a * 1e-6) / 1e9:.0f} GB/s at the "
        f"average duration ({nb / (a * 1e-6) / 1e9 / PEAK_HBM_GBS * 100:.1f}% of 8 TB/s); HBM read "
        f"{rb / 1e6:.1f} MB, written {wb / 1e6:.1f} MB (FETCH_SIZE / WRITE_SIZE scaled by a 1 GiB copy)."
        for n, c, a, mn_, mx_, nb, what, rb, wb in lines)
    md = f"""# Row softmax (online normaliser) and fused softmax top-k on 512 rows of 256000 fp32 logits (k = 8)

Command (run from the repository root on one MI355X):

    {cmds["trace_softmax"]}

Kernel trace statistics (`run_kernel_stats.csv`; warm-up included):

| kernel | calls | average (us) | min (us) | max (us) |
|---|---|---|---|---|
{table}

{detail}

The softmax's read bytes are about twice x: FETCH_SIZE counts every read
that misses the L2, whether the Infinity Cache (256 MB, memory side) or HBM
serves it.  x (524 MB) exceeds that cache, but the second read walks each
row backwards and finds the part read last in pass 1 still cached; the
counters cannot show this, the kernel time does (284 us with a forward
second read and non-temporal first read, 245 us now).
"""
    with open(os.path.join(ROOT, "profiles", "softmax_fp32_rows512_n256000.md"), "w") as f:
        f.write(md)
    print(json.dumps({k: traffic[k]["bytes_per_launch"] for k in ("prefill", "decode", "combine", "prefill_fp8",
                                                                  "rolling_decode", "softmax", "topk")}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed launches of each leg for this much wall time before its warm-up")
    ap.add_argument("--workload", choices=["prefill", "decode", "prefill_fp8", "rolling", "softmax"],
                    default="prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="prefill leg only (no other legs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (for scaling HBM byte counters)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="host only: write profiles/ from the rocprofv3 output under DIR")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").random_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 3}))
        return
    import online_softmax_tiled_amd as fa
    fa.load_library()
    torch.cuda.init()
    K, W, settle = args.steps, args.warmup, args.settle_ms

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---- every leg's inputs generated and uploaded before any timing
    wk = args.workload
    all_legs = wk == "prefill" and not args.no_decode
    prep = {}
    if wk == "prefill":
        prep["prefill"] = prepare_prefill(torch, fa)
    if wk == "decode" or all_legs:
        prep["decode"] = prepare_decode(torch, fa)
    if wk == "rolling" or all_legs:
        prep["rolling"] = prepare_rolling(torch, fa)
    if wk == "softmax" or all_legs:
        prep["softmax"] = prepare_softmax(torch, fa)
    if wk == "prefill_fp8" or all_legs:
        prep["prefill_fp8"] = prepare_prefill_fp8(torch, fa)
    if all_legs:
        for name in OTHER_PREFILL:
            prep[name] = prepare_prefill(torch, fa, name)
        prep["standard_attention"] = prepare_standard_attention(torch)
    torch.cuda.synchronize()
    log("inputs of every leg resident in HBM")

    def run(parts):
        return time_leg(parts, K, W, settle, torch)

    out_legs = {}
    if "prefill" in prep:
        w, parts = prep["prefill"]
        t = run(parts)
        flops = wl.algorithmic_flops(w)
        mean = t.per_step(K)  # one kernel per step: its average launch duration over the timed region
        out_legs["prefill"] = (w, t, {
            "value": flops * K / (t.total_ms * 1e-3) / 1e12, "unit": "TFLOP/s",
            "timing": Timing.stats(t.part_ms[0]),
            "roofline": {"bound": "mfma", "achieved": round(flops / (mean * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops / (mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic("prefill")}})
        log(f"prefill done: {t.per_step(K):.4f} ms/launch (median {np.median(t.part_ms[0]):.4f})")
    if "decode" in prep:
        w, parts = prep["decode"]
        t = run(parts)
        nbytes = wl.algorithmic_bytes(w)
        S = w.num_splits
        part_bytes = w.B * w.H * w.Nq * S * (w.d + 2) * 4
        split_bytes = nbytes - part_bytes - (w.B * w.H * w.Nq * (w.d * 2 + 4))  # q, k, v in; partials out
        split_mean = float(np.mean(t.part_ms[0]))
        value = nbytes * K / (t.total_ms * 1e-3) / 1e9
        out_legs["decode"] = (w, t, {
            "workload": w.name, "value": round(value, 1), "unit": "GB/s",
            "ms_per_step": round(t.per_step(K), 4), "frac_of_hbm_peak": round(value / PEAK_HBM_GBS, 4),
            "timing": {"step": Timing.stats(t.step_ms), "split_kernel": Timing.stats(t.part_ms[0]),
                       "combine_kernel": Timing.stats(t.part_ms[1])},
            "step_frac_of_hbm_peak_at_median": round(nbytes / (np.median(t.step_ms) * 1e-3) / 1e9
                                                     / PEAK_HBM_GBS, 4),
            "roofline": {"bound": "hbm", "achieved": round(split_bytes / (split_mean * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(split_bytes / (split_mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("decode"), "kernel": "splitkv_decode_kernel",
                         "avg_ms": round(split_mean, 4)}})
        log(f"decode done: {t.per_step(K):.4f} ms/step (median {np.median(t.step_ms):.4f})")
    if "rolling" in prep:
        w, parts = prep["rolling"]
        t = run(parts)
        nbytes = wl.rolling_bytes(w)
        S = w.num_splits
        dec_bytes = 2 * w.rows * w.B * w.Hkv * w.d * 2 + w.B * w.H * w.d * 2 + w.B * w.H * S * (w.d + 2) * 4
        dec_mean = float(np.mean(t.part_ms[1]))
        value = nbytes * K / (t.total_ms * 1e-3) / 1e9
        out_legs["rolling"] = (w, t, {
            "workload": w.name, "value": round(value, 1), "unit": "GB/s",
            "ms_per_step": round(t.per_step(K), 4), "frac_of_hbm_peak": round(value / PEAK_HBM_GBS, 4),
            "config": {"B": w.B, "H": w.H, "Hkv": w.Hkv, "d": w.d, "window": w.window, "sinks": w.sinks,
                       "pos": w.pos, "cache_rows_read": w.rows, "num_splits": S},
            "timing": {"step": Timing.stats(t.step_ms), "append_kernel": Timing.stats(t.part_ms[0]),
                       "decode_kernel": Timing.stats(t.part_ms[1]), "combine_kernel": Timing.stats(t.part_ms[2])},
            "roofline": {"bound": "hbm", "achieved": round(dec_bytes / (dec_mean * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(dec_bytes / (dec_mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("rolling_decode"),
                         "kernel": "splitkv_decode_kernel (rolling cache)", "avg_ms": round(dec_mean, 4)}})
        log(f"rolling decode done: {t.per_step(K):.4f} ms/step")
    if "softmax" in prep:
        w, legs = prep["softmax"]
        b = wl.softmax_bytes(w)
        res = {n: run(p) for n, p in legs.items()}
        sm = {"workload": w.name, "config": {"rows": w.rows, "n": w.n, "k": w.k, "dtype": "fp32"}}
        for name, nbytes in (("softmax", b["softmax_online"]), ("topk", b["topk_fused"])):
            t = res[name]
            mean = t.per_step(K)
            gbs = nbytes / (mean * 1e-3) / 1e9
            sm[name] = {"ms_per_step": round(t.per_step(K), 4), "timing": Timing.stats(t.part_ms[0]),
                        "bytes": nbytes, "value": round(gbs, 1), "unit": "GB/s",
                        "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic(name)}
        ts, tt = (float(np.median(res[n].step_ms)) for n in ("torch_softmax", "torch_softmax_topk"))
        sm["softmax"]["bytes_note"] = "two reads of x and one write of y (online normaliser)"
        sm["softmax"]["byte_ratio_vs_three_pass"] = round(b["softmax_three_pass"] / b["softmax_online"], 3)
        sm["softmax"]["torch_softmax_median_ms"] = round(ts, 4)
        sm["softmax"]["speedup_vs_torch"] = round(ts / float(np.median(res["softmax"].part_ms[0])), 3)
        sm["topk"]["bytes_note"] = "one read of x; k probabilities and indices written"
        unfused = b["softmax_three_pass"] + w.rows * w.n * 4 + w.rows * w.k * 8
        sm["topk"]["byte_ratio_vs_unfused"] = round(unfused / b["topk_fused"], 3)
        sm["topk"]["torch_softmax_topk_median_ms"] = round(tt, 4)
        sm["topk"]["speedup_vs_torch"] = round(tt / float(np.median(res["topk"].part_ms[0])), 3)
        out_legs["softmax"] = (w, None, sm)
        log(f"softmax done: {sm['softmax']['ms_per_step']:.4f} ms, top-k {sm['topk']['ms_per_step']:.4f} ms")
    if "prefill_fp8" in prep:
        w, parts = prep["prefill_fp8"]
        t = run(parts)
        flops = wl.algorithmic_flops(w)
        mean = t.per_step(K)
        value = flops * K / (t.total_ms * 1e-3) / 1e12
        out_legs["prefill_fp8"] = (w, t, {
            "workload": w.name, "value": round(value, 2), "unit": "TFLOP/s", "ms_per_step": round(t.per_step(K), 4),
            "dtype": "fp8 e4m3 (bf16 out)", "timing": Timing.stats(t.part_ms[0]),
            "roofline": {"bound": "mfma", "achieved": round(flops / (mean * 1e-3) / 1e12, 2),
                         "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops / (mean * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                         "traffic": measured_traffic("prefill_fp8")}})
        log(f"fp8 prefill done: {t.per_step(K):.4f} ms/launch")
    others = {}
    for name in OTHER_PREFILL:
        if name not in prep:
            continue
        w, parts = prep[name]
        t = run(parts)
        flops = wl.algorithmic_flops(w)
        value = flops * K / (t.total_ms * 1e-3) / 1e12
        others[name] = {"workload": name, "value": round(value, 2), "unit": "TFLOP/s",
                        "ms_per_step": round(t.per_step(K), 4), "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
                        "timing": Timing.stats(t.part_ms[0]),
                        "config": {"B": w.B, "H": w.H, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                                   "causal": w.causal, "head_window": "W on even heads" if w.head_window else None,
                                   "softcap": w.softcap or None}}
        log(f"{name} done: {t.per_step(K):.4f} ms/launch")
    std = None
    if "standard_attention" in prep:
        w, parts = prep["standard_attention"]
        t = time_leg(parts, 3, 1, 0.0, torch)
        std = {"workload": w.name + " (first batch element)", "median_ms": round(float(np.median(t.step_ms)), 4)}
        del prep["standard_attention"]
        torch.cuda.empty_cache()
        log(f"standard attention done: {std['median_ms']:.3f} ms")
    dev = device_info(torch)
    log("device info done")

    main_key = {"prefill": "prefill", "decode": "decode", "prefill_fp8": "prefill_fp8", "rolling": "rolling",
                "softmax": "softmax"}[wk]
    if wk in ("rolling", "softmax"):
        print(json.dumps({"leg": wk, **out_legs[main_key][2]}), flush=True)
        return
    w, t, leg = out_legs[main_key]
    out = {
        "metric": METRIC, "value": round(leg["value"], 2), "unit": leg["unit"], "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(t.per_step(K), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8" if wk == "prefill_fp8" else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "num_splits": w.num_splits or None, "parallelism": "none (1 GPU)"},
        "timing": {"per_launch": leg["timing"] if "step" not in leg.get("timing", {}) else leg["timing"]["step"],
                   "settle_ms": settle,
                   "method": "value and ms_per_step: one pair of HIP events on the launch stream around the "
                             "K back-to-back timed steps; per_launch: a second pass of K steps with events "
                             "before and after every kernel; before its warm-up each leg runs untimed for "
                             "settle_ms of wall time (an idle GPU needs tens of milliseconds to reach its "
                             "working clock)"},
        "roofline": leg["roofline"],
    }
    if wk == "prefill" and std is not None:
        ours_b1 = float(np.median(t.part_ms[0])) / w.B
        std["ours_median_ms_per_batch_element"] = round(ours_b1, 4)
        std["speedup"] = round(std["median_ms"] / ours_b1, 2)
        out["standard_attention"] = std
    for key in ("decode", "rolling", "softmax", "prefill_fp8"):
        if key in out_legs and key != main_key:
            out[key] = out_legs[key][2]
    if others:
        out["other_prefill"] = others
    out["device"] = dev
    out["pages_context"] = PAGES_CONTEXT
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
        log("cpu baseline done")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
