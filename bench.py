"""Benchmark of the fused no-KV-cache attention forward on one MI355X.

One step = one mha_no_cache call over the whole workload (all query tiles,
all heads, all batches), inputs already resident in HBM. Prints ONE JSON
line. Default workload: batch 2, 4096 tokens, 32 query heads sharing 8 K/V
heads, head dim 128, bf16, causal mask, scale 1/sqrt(128).

Metric: attention forward TFLOP/s counting only unmasked (query, key)
pairs, FLOP = 4 * D * visible_pairs * B * H, and that rate as a fraction of
MI355X's dense bf16/fp16 MFMA peak (2516.6 TFLOP/s).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--all]
                  [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}  # dense MFMA, MI355X spec
METRIC = "attention fwd TFLOP/s (unmasked FLOPs) + % of MFMA bf16 peak, 1×MI355X"
DEFAULT_WORKLOAD = "gqa_b2_s4096_h32kv8_d128_bf16_causal"
KERNEL_NAME = "mha_fwd"


def visible_pairs(S: int, mask: str, window: int) -> int:
    """Closed-form count of (query, key) pairs a mask leaves visible in one head."""
    if mask == "none":
        return S * S
    if mask == "causal":
        return S * (S + 1) // 2
    w = min(window, S)
    return S * w - w * (w - 1) // 2


def flops(w) -> int:
    return 4 * w.D * visible_pairs(w.S, w.mask, w.window) * w.B * w.H


def algorithmic_bytes(w) -> int:
    e = 4 if w.dtype == "f32" else 2
    return e * w.B * w.S * w.D * (2 * w.H + 2 * w.Hkv)  # Q, O, K, V once each


SETTLE_S = 0.3
SPEC_SCLK_MHZ = 2400  # shader clock the spec MFMA peak assumes


def _gpu_sysfs_dir():
    """sysfs directory of the first amdgpu device with a shader-clock table."""
    import glob

    for d in sorted(glob.glob("/sys/class/drm/card*/device")):
        if os.path.isfile(os.path.join(d, "pp_dpm_sclk")):
            return d
    return None


class ClockSampler:
    """Samples the shader clock (MHz: the pp_dpm_sclk level marked current)
    and the socket power (W: hwmon power1_input) from sysfs in a background
    thread while the GPU runs. Reading sysfs does not touch the GPU's queues.
    Without those files (not an amdgpu host) it records nothing."""

    def __init__(self, period_s: float = 0.02):
        self.dir = _gpu_sysfs_dir()
        self.power_file = self.cap_w = None
        if self.dir:
            import glob

            for h in sorted(glob.glob(os.path.join(self.dir, "hwmon", "hwmon*"))):
                if os.path.isfile(os.path.join(h, "power1_input")):
                    self.power_file = os.path.join(h, "power1_input")
                    cap = os.path.join(h, "power1_cap")
                    if os.path.isfile(cap):
                        self.cap_w = int(open(cap).read()) / 1e6
                    break
        self.period = period_s
        self.samples = []  # (time.perf_counter(), MHz or None, W or None)
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        mhz = None
        with open(os.path.join(self.dir, "pp_dpm_sclk")) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*mhz", line, re.I)
                    mhz = int(m.group(1)) if m else None
        watts = int(open(self.power_file).read()) / 1e6 if self.power_file else None
        return mhz, watts

    def _run(self):
        while not self._stop.is_set():
            try:
                mhz, watts = self._read()
            except (OSError, ValueError):
                return
            self.samples.append((time.perf_counter(), mhz, watts))
            self._stop.wait(self.period)

    def start(self):
        if self.dir:
            self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self, t_from: float = 0.0):
        """Medians over the samples taken at or after t_from, or None."""
        ss = [x for x in self.samples if x[0] >= t_from]
        mhz = sorted(x[1] for x in ss if x[1] is not None)
        watts = sorted(x[2] for x in ss if x[2] is not None)
        if not mhz:
            return None
        return {"sclk_mhz": mhz[len(mhz) // 2],
                "power_w": round(watts[len(watts) // 2], 1) if watts else None,
                "power_cap_w": self.cap_w, "samples": len(mhz)}


def time_gpu(w, steps: int, warmup: int):
    import torch

    import head_attention_no_amd as fa
    from head_attention_no_amd import inputs

    q, k, v = inputs.workload_qkv(w)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    # The GPU raises its clock over the first tens of milliseconds of load:
    # launch back-to-back for SETTLE_S seconds before the counted warmup so
    # the timed steps see the steady state (measured: the first ~40 launches
    # of this kernel run ~12% slower than later ones).
    # The shader clock is sampled over the settled part of that period.
    sampler = ClockSampler().start()
    t_start = time.perf_counter()
    t_end = t_start + SETTLE_S
    while time.perf_counter() < t_end:
        for _ in range(8):
            fa.attention(q, k, v, w.scale, w.mask, w.window, out=out, stream=stream)
        torch.cuda.synchronize()
    sampler.stop()
    clock = sampler.summary(t_start + SETTLE_S / 3)
    for _ in range(warmup):
        fa.attention(q, k, v, w.scale, w.mask, w.window, out=out, stream=stream)
    torch.cuda.synchronize()
    # The timed steps: one pair of HIP events around them on the kernel's
    # stream (no event between launches), bracketed by synchronisations.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fa.attention(q, k, v, w.scale, w.mask, w.window, out=out, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = e0.elapsed_time(e1)
    # Spread of single launches (each between two events), after the timed
    # steps; reported beside the mean, not used for it.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for s, e in ev:
        s.record(stream)
        fa.attention(q, k, v, w.scale, w.mask, w.window, out=out, stream=stream)
        e.record(stream)
    torch.cuda.synchronize()
    launch_ms = sorted(s.elapsed_time(e) for s, e in ev)
    return {
        "wall_s": wall,
        "ms_per_step": wall * 1e3 / steps,
        "launch_ms_mean": region_ms / steps,
        "launch_ms_median": launch_ms[len(launch_ms) // 2],
        "launch_ms_min": launch_ms[0],
        "single_launch_ms_mean": sum(launch_ms) / len(launch_ms),
        "clock": clock,
    }


FLUSH_MIB = 512  # larger than the L2s (4 MiB per XCD) and the 256 MiB MALL together


def time_cold(w, steps: int):
    """The kernel with cold caches: before each launch a 512 MiB buffer is
    written, which evicts q, k, v and out from the L2s and the MALL; HIP
    events on the kernel's stream bracket the launch alone."""
    import torch

    import head_attention_no_amd as fa
    from head_attention_no_amd import inputs

    q, k, v = (x.cuda() for x in inputs.workload_qkv(w))
    out = torch.empty_like(q)
    flush = torch.empty(FLUSH_MIB << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i, (s, e) in enumerate(ev):
        flush.fill_(i & 0xFF)
        s.record(stream)
        fa.attention(q, k, v, w.scale, w.mask, w.window, out=out, stream=stream)
        e.record(stream)
    torch.cuda.synchronize()
    ms = sorted(s.elapsed_time(e) for s, e in ev)
    mean = sum(ms) / len(ms)
    return {"launches": steps, "flush_bytes_before_each": FLUSH_MIB << 20,
            "launch_ms_mean": round(mean, 5), "launch_ms_median": round(ms[len(ms) // 2], 5),
            "tflops_mean": round(flops(w) / (mean * 1e-3) / 1e12, 2)}


def cpu_baseline(w, budget_s: float = 12.0):
    """The fp64 oracle on a bounded sample: whole K/V head groups (one K/V
    head and its H/Hkv query heads), batch by batch, until the time budget is
    spent or the workload is done."""
    import oracle
    from head_attention_no_amd import inputs

    q, k, v = inputs.workload_qkv(w)
    rep = w.H // w.Hkv
    orc = oracle.default()
    done, t_total = 0, 0.0
    for b in range(w.B):
        for g in range(w.Hkv):
            qs = q[b:b + 1, :, g * rep:(g + 1) * rep].contiguous()
            ks, vs = k[b:b + 1, :, g:g + 1].contiguous(), v[b:b + 1, :, g:g + 1].contiguous()
            t0 = time.perf_counter()
            orc.attention(qs, ks, vs, w.scale, w.mask, w.window)
            t_total += time.perf_counter() - t0
            done += 1
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    sample_flop = 4 * w.D * visible_pairs(w.S, w.mask, w.window) * rep * done
    return {
        "value": sample_flop / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": orc.threads(),
        "kind": "oracle",
        "sample": f"{done * rep} of {w.B * w.H} (batch, head) pairs, in batch order "
                  f"({done} K/V group(s) x {rep} query heads), full S={w.S} rows; "
                  f"{t_total:.1f} s fp64 on {orc.threads()} threads "
                  f"({platform.processor() or platform.machine()})",
        "seconds": t_total,
    }


def copy_calibration(mib: int, steps: int, warmup: int):
    """A plain device-to-device copy of known size: its HBM counters per
    dispatch calibrate the ones read for the attention kernel."""
    import torch

    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    return {"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": ms,
            "GBps_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}


def yardsticks(w, steps: int, warmup: int):
    """Context for the roofline fraction, on the same GPU: a large bf16 GEMM
    through torch.matmul (hipBLASLt) and torch's fused attention (its flash
    backend only, so it raises rather than fall back to the unfused math
    path) on workload w, both timed like the kernel."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    from head_attention_no_amd import inputs

    def timed(fn):
        t_end = time.perf_counter() + SETTLE_S
        while time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps

    out = {}
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    ms = timed(lambda: torch.matmul(a, b))
    out["gemm_bf16_8192"] = {"ms": round(ms, 4), "tflops": round(2 * n ** 3 / ms / 1e9, 1)}
    del a, b
    q, k, v = (t.cuda() for t in inputs.workload_qkv(w))
    rep = w.H // w.Hkv
    # BSHD -> BHSD views made contiguous; K/V heads repeated for the grouped case.
    qh = q.transpose(1, 2).contiguous()
    kh = k.transpose(1, 2).repeat_interleave(rep, dim=1).contiguous()
    vh = v.transpose(1, 2).repeat_interleave(rep, dim=1).contiguous()
    if w.mask == "causal":
        try:
            with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
                ms = timed(lambda: F.scaled_dot_product_attention(qh, kh, vh, is_causal=True,
                                                                  scale=w.scale))
            out["torch_sdpa_flash"] = {"ms": round(ms, 4), "tflops": round(flops(w) / ms / 1e9, 1)}
        except RuntimeError as ex:
            out["torch_sdpa_flash"] = {"unavailable": str(ex)[:200]}
    return {"workload": w.name, "yardsticks": out}


# Sources of the attention path (the top-K kernel is not part of it).
ATTENTION_SOURCES = ("fa355.hip", "mha_common.hpp", "mha_fwd16.hpp", "mha_fwd32.hpp", "mha_launch.hip",
                     "mha_launch.hpp")


def kernel_sources_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for name in ATTENTION_SOURCES:
        with open(os.path.join(ROOT, "head_attention_no_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(w):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counter
    runs (profiles/*.traffic.json), scaled by a plain copy's counters; None
    when no file covers this workload or the kernel sources changed since."""
    import glob

    cur = kernel_sources_hash()
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.traffic.json"))):
        with open(f) as fh:
            d = json.load(fh)
        if d.get("workload") == w.name and d.get("kernel_sources_sha256_16") == cur:
            return int(d["traffic_bytes_per_launch"]), os.path.basename(f)
    return None, None


def write_traffic(w, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str):
    """Writes profiles/<kernel>_<workload>.traffic.json from four rocprofv3
    --pmc runs (FETCH_SIZE and WRITE_SIZE of the workload's bench run, and of
    the --copy-calibration 256 run): the last attention dispatch's counters,
    each scaled by what the same counter reads for the plain 256 MiB copy."""
    import csv

    def last(d, name_part):
        with open(os.path.join(d, "pmc_counter_collection.csv")) as fh:
            rows = [r for r in csv.DictReader(fh) if name_part in r["Kernel_Name"]]
        did = max(int(r["Dispatch_Id"]) for r in rows)
        return {r["Counter_Name"]: float(r["Counter_Value"]) for r in rows if int(r["Dispatch_Id"]) == did}

    fetch = last(fetch_dir, "mha_fwd")["FETCH_SIZE"]
    write = last(write_dir, "mha_fwd")["WRITE_SIZE"]
    cf = last(copy_fetch_dir, "copyBuffer")["FETCH_SIZE"]
    cw = last(copy_write_dir, "copyBuffer")["WRITE_SIZE"]
    fs, ws = 256 * 1024 / cf, 256 * 1024 / cw
    name = f"mha_fwd16_{w.dtype}_d{w.D}_{w.mask}_{w.name.split('_', 1)[1]}" if w.dtype != "f32" else w.name
    out = {"kernel_sources_sha256_16": kernel_sources_hash(), "workload": w.name,
           "fetch_kib": fetch, "write_kib": write, "fetch_scale": fs, "write_scale": ws,
           "traffic_bytes_per_launch": fetch * 1024 * fs + write * 1024 * ws}
    path = os.path.join(ROOT, "profiles", f"{TRAFFIC_FILE.get(w.name, name)}.traffic.json")
    out["source"] = os.path.basename(path).replace(".traffic.json", ".md")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    return path, out


# Profile file stem per workload (the bench workload's profile name).
TRAFFIC_FILE = {"gqa_b2_s4096_h32kv8_d128_bf16_causal": "mha_fwd16_bf16_d128_causal_gqa_b2_s4096"}


def roofline(w, t):
    fl = flops(w)
    achieved = fl / (t["launch_ms_mean"] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic, src = measured_traffic(w)
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic, "traffic_unit": "bytes/launch",
            "traffic_source": src, "kernel": KERNEL_NAME, "flop_per_launch": fl,
            "launch_ms_mean": round(t["launch_ms_mean"], 5)}


HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, spec


def time_topk(steps: int, warmup: int, with_cpu: bool):
    """The top-K ordering kernel on its workload (rows of next-token
    frequencies): HBM-bound, so reported as GB/s of algorithmic traffic
    (the input read once, values and indices written once) against the HBM
    peak, plus the oracle on a sample of rows."""
    import torch

    import head_attention_no_amd as fa
    from head_attention_no_amd import inputs

    w = inputs.TOPK_WORKLOAD
    x_cpu = inputs.make_scores(w["B"], w["V"], w["kind"], seed=w["seed"])
    x = x_cpu.cuda()
    vals = torch.empty(w["B"], w["K"], device="cuda")
    idx = torch.empty(w["B"], w["K"], dtype=torch.int32, device="cuda")
    call = lambda: fa.topk(x, w["K"], values=vals, indices=idx)  # noqa: E731

    def per_launch_ms(fn):
        """Mean per launch over `steps` back-to-back launches between one
        pair of HIP events (after a settle period and warm-up)."""
        t_end = time.perf_counter() + SETTLE_S
        while time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps

    ms = per_launch_ms(call)
    nbytes = w["B"] * w["V"] * 4 + w["B"] * w["K"] * 8
    gbps = nbytes / (ms * 1e-3) / 1e9
    out = {"workload": w["name"], "launch_ms_mean": round(ms, 5),
           "rows_per_s": round(w["B"] / (ms * 1e-3), 1),
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                        "algorithmic_bytes": nbytes}}
    # Yardsticks, timed the same way: the library top-K on the same rows,
    # and a plain streaming read of them (a row max), the floor for one read.
    ms_lib = per_launch_ms(lambda: torch.topk(x, w["K"], dim=1))
    ms_read = per_launch_ms(lambda: torch.amax(x, dim=1))
    out["yardsticks"] = {"torch_topk": {"launch_ms_mean": round(ms_lib, 5)},
                         "torch_row_max_read": {"launch_ms_mean": round(ms_read, 5),
                                                "gbps": round(w["B"] * w["V"] * 4 / (ms_read * 1e-3) / 1e9, 1)}}
    if with_cpu:
        from oracle import topk as otk

        n = 16
        t0 = time.perf_counter()
        otk.topk_rows(x_cpu[:n].numpy(), w["K"])
        sec = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(n / sec, 1), "unit": "rows/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{n} of {w['B']} rows, numpy lexsort per row, {sec:.2f} s"}
    return out


def one_line(w, args, t, cpu):
    fl = flops(w)
    tflops = fl / (t["ms_per_step"] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    return {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(t["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "H": w.H, "Hkv": w.Hkv, "D": w.D,
                   "mask": w.mask, "window": w.window, "scale": w.scale,
                   "flop_per_step": fl, "algorithmic_bytes_per_step": algorithmic_bytes(w)},
        "pct_of_mfma_peak": round(100 * tflops / peak, 2),
        "roofline": roofline(w, t),
        "clock": clock_context(fl, t, peak),
        "cpu_baseline": cpu,
    }


def clock_context(fl, t, peak):
    """The shader clock under this load and the MFMA peak at that clock: the
    spec peak assumes 2.4 GHz, and the GPU lowers its clock to stay within
    its power cap."""
    c = t.get("clock")
    if not c:
        return None
    at = peak * c["sclk_mhz"] / SPEC_SCLK_MHZ
    achieved = fl / (t["launch_ms_mean"] * 1e-3) / 1e12
    return dict(c, peak_at_sclk_tflops=round(at, 1), frac_at_sclk=round(achieved / at, 4))


def sustained_clocks(names, seconds: float):
    """Each workload (and a bf16 8192^3 GEMM through torch.matmul) launched
    back-to-back for `seconds`, with the shader clock and socket power sampled
    over the last two thirds of the run."""
    import torch

    import head_attention_no_amd as fa
    from head_attention_no_amd import inputs

    def run(fn, launches_per_batch):
        sampler = ClockSampler().start()
        t0 = time.perf_counter()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 0
        while time.perf_counter() - t0 < seconds:
            s.record()
            for _ in range(launches_per_batch):
                fn()
            e.record()
            torch.cuda.synchronize()
            n += launches_per_batch
        sampler.stop()
        return s.elapsed_time(e) / launches_per_batch, n, sampler.summary(t0 + seconds / 3)

    out = {}
    for name in names:
        w = inputs.BY_NAME[name]
        q, k, v = (x.cuda() for x in inputs.workload_qkv(w))
        o = torch.empty_like(q)
        ms, n, c = run(lambda: fa.attention(q, k, v, w.scale, w.mask, w.window, out=o), 20)
        tf = flops(w) / ms / 1e9
        out[name] = {"launch_ms": round(ms, 5), "launches": n, "tflops": round(tf, 1),
                     "frac_of_peak": round(tf / PEAK_TFLOPS[w.dtype], 4), "clock": c}
        if c:
            out[name]["frac_at_sclk"] = round(
                tf / (PEAK_TFLOPS[w.dtype] * c["sclk_mhz"] / SPEC_SCLK_MHZ), 4)
        del q, k, v, o
    n3 = 8192
    a = torch.randn(n3, n3, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n3, n3, device="cuda", dtype=torch.bfloat16)
    ms, n, c = run(lambda: torch.matmul(a, b), 5)
    tf = 2 * n3 ** 3 / ms / 1e9
    out["gemm_bf16_8192"] = {"launch_ms": round(ms, 5), "launches": n, "tflops": round(tf, 1),
                             "frac_of_peak": round(tf / PEAK_TFLOPS["bf16"], 4), "clock": c}
    if c:
        out["gemm_bf16_8192"]["frac_at_sclk"] = round(
            tf / (PEAK_TFLOPS["bf16"] * c["sclk_mhz"] / SPEC_SCLK_MHZ), 4)
    return {"sustained_s": seconds, "results": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--all", action="store_true",
                    help="also time the other workloads (reported under 'other_workloads')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--yardstick", action="store_true",
                    help="instead, time a large bf16 GEMM and torch's flash attention on the "
                         "workload, for context")
    ap.add_argument("--topk", action="store_true",
                    help="instead, time only the top-K ordering kernel on its workload")
    ap.add_argument("--clocks", type=float, default=0.0, metavar="SECONDS",
                    help="instead, run the workload (with --all: every workload) and a bf16 "
                         "GEMM back-to-back for SECONDS each, sampling shader clock and power")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead, time a plain device copy of MIB MiB (reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="instead, write profiles/*.traffic.json for --workload from four rocprofv3 "
                         "--pmc output folders (no GPU needed)")
    args = ap.parse_args()
    if args.write_traffic:
        from head_attention_no_amd import inputs as _inputs

        path, out = write_traffic(_inputs.BY_NAME[args.workload], *args.write_traffic)
        print(path, json.dumps(out))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the kernel needs no "
              "collective, and this build measures a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch

    from head_attention_no_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(args.copy_calibration, args.steps, args.warmup)))
        return
    if args.topk:
        print(json.dumps(time_topk(args.steps, args.warmup, not args.no_cpu_baseline)))
        return
    w = inputs.BY_NAME[args.workload]
    if args.clocks:
        names = [w.name] + ([o.name for o in inputs.WORKLOADS + inputs.WIDER if o.name != w.name]
                            if args.all else [])
        print(json.dumps(sustained_clocks(names, args.clocks)), flush=True)
        return
    if args.yardstick:
        print(json.dumps(yardsticks(w, args.steps, args.warmup)))
        return
    print(f"# timing {w.name}: {args.warmup} warmup + {args.steps} steps", file=sys.stderr,
          flush=True)
    t = time_gpu(w, args.steps, args.warmup)
    cold = time_cold(w, max(10, min(args.steps, 30)))
    line = None
    cpu = None
    if not args.no_cpu_baseline:
        print("# cpu baseline (fp64 oracle sample)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w)
    line = one_line(w, args, t, cpu)
    line["cold_cache"] = cold
    if args.all:
        others = {}
        for o in inputs.WORKLOADS + inputs.WIDER:
            if o.name == w.name:
                continue
            print(f"# timing {o.name}", file=sys.stderr, flush=True)
            to = time_gpu(o, args.steps, args.warmup)
            fo = flops(o)
            others[o.name] = {
                "ms_per_step": round(to["ms_per_step"], 5),
                "tflops": round(fo / (to["ms_per_step"] * 1e-3) / 1e12, 2),
                "launch_ms_mean": round(to["launch_ms_mean"], 5),
                "pct_of_peak": round(100 * fo / (to["launch_ms_mean"] * 1e-3) / 1e12
                                     / PEAK_TFLOPS[o.dtype], 2),
                "peak_tflops": PEAK_TFLOPS[o.dtype],
            }
        line["other_workloads"] = others
        print("# timing top-K ordering", file=sys.stderr, flush=True)
        line["topk"] = time_topk(args.steps, args.warmup, not args.no_cpu_baseline)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
