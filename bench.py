#!/usr/bin/env python3
"""Attention-forward throughput on one MI355X.

One step = one fa_fwd_ex call over the whole batch of the workload (every
stage of the forward pass runs inside that launch).  Inputs are seeded
synthetic tensors already resident in HBM when the timed region starts.

Prints ONE JSON line with the throughput (attention TFLOP/s, FLOPs =
4*B*H*N_q*N_kv*d, halved for causal), the dominant kernel's roofline
position (algorithmic FLOPs per launch / average launch time from HIP
events on the launch stream, against the bf16/fp16/fp8/fp32 dense MFMA
peak) and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("attention fwd TFLOP/s (4·B·H·N²·d) and % of MFMA peak, "
          "bf16 N=8K d=128")
BWD_METRIC = "attention bwd TFLOP/s (10·B·H·N²·d: S, dP, dV, dK, dQ) and % of MFMA peak"
DEFAULT_WORKLOAD = "headline_bf16_n8192_d128"
# MI355X dense peaks, TFLOP/s: 256 CUs x 2.4 GHz x flop/clk/CU of the matrix cores
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "fp8_e4m3": 5033.2, "f32": 157.3}
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
ELEM_BYTES = {"bf16": 2, "f16": 2, "fp8_e4m3": 1, "f32": 4}


def algorithmic_bytes_bwd(w) -> float:
    """Backward: Q, K, V, O, dO and LSE read once; dQ, dK, dV written once."""
    e = ELEM_BYTES[w.dtype]
    return float(w.B * w.H * ((4 * w.n_q + 4 * w.n_kv) * w.d * e + 8 * w.n_q))


def algorithmic_bytes(w) -> float:
    """Q, K, V read once; O and LSE written once (bytes per launch)."""
    e = ELEM_BYTES[w.dtype]
    oe = 2 if w.dtype == "fp8_e4m3" else e
    per_head = (w.n_q * w.d * e + 2 * w.n_kv * w.d * e + w.n_q * w.d * oe + w.n_q * 4)
    return float(w.B * w.H * per_head)
def materialised_bytes(w) -> float:
    """HBM bytes of the standard three-step method ("FlashAttention 与显存",
    plates 04 and 14): Q, K, V read and O written once, and the N_q x N_kv
    matrices S and P each written once and read once, all in the input's
    element size."""
    e = ELEM_BYTES[w.dtype]
    return float(w.B * w.H * e * ((2 * w.n_q + 2 * w.n_kv) * w.d + 4 * w.n_q * w.n_kv))


def fa_bytes_without_l2(w, br: int) -> float:
    """HBM bytes of the tiled method with no cache reuse ("FlashAttention 与显存",
    plate 14, second-version order): each block of br query rows is read once
    and reads all of K and V once; O is written once."""
    e = ELEM_BYTES[w.dtype]
    passes = -(-w.n_q // br)
    return float(w.B * w.H * e * (2 * w.n_q * w.d + passes * 2 * w.n_kv * w.d))


def variant_rows(name: str) -> int:
    """Query rows per workgroup of a variant named br<waves>x<rows per wave>_..."""
    import re
    m = re.search(r"br(\d+)x(\d+)", name)
    if not m:
        raise ValueError("variant name without a row block: %r" % name)
    return int(m.group(1)) * int(m.group(2))


TRAFFIC_DIR = os.path.join(ROOT, "profiles")


KERNEL_SOURCE = {"f32": "fa_fwd32.hip", "f16": "fa_fwd16.hip", "bf16": "fa_fwd16.hip",
                 "fp8_e4m3": "fa_fwd8.hip"}


def kernel_source_digest(dtype: str, bwd: bool = False) -> str:
    """Hash of the device sources that make the workload's kernels (its .hip
    file and the shared device and tile headers), to tell whether stored
    counters still apply.  Host code (validation, variant table) is left out:
    the stored record names the variant it was taken on instead."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_95_amd", "csrc")
    names = ["fa_device.h", "fa_internal.h", "fa_bwd16.hip" if bwd else KERNEL_SOURCE[dtype]]
    if bwd or dtype in ("f16", "bf16"):
        names.append("fa_tile16.h")
    for name in sorted(names):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, dtype: str, variant: str, bwd: bool = False):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources and the same variant; else None."""
    path = os.path.join(TRAFFIC_DIR, "traffic_%s%s.json" % (workload, "_bwd" if bwd else ""))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_digest") != kernel_source_digest(dtype, bwd):
        return None
    if rec.get("variant") != variant:
        return None
    return rec.get("hbm_bytes_per_launch")


def variant_label(workload: str, tile: int = 0, splitkv=None, bwd: bool = False) -> str:
    """The launch configuration a bench run of the workload times: the
    backward, split-KV, or the forward tile variant's name (host-only)."""
    from exact_attention_95_amd import fa
    from exact_attention_95_amd.inputs import WORKLOADS
    w = WORKLOADS[workload]
    if bwd:
        return "backward"
    if splitkv is None and w.n_q <= 16:
        splitkv = 0
    if splitkv is not None and splitkv >= 0:
        return "split_kv(%s)" % ("auto" if splitkv == 0 else splitkv)
    code = {"f32": fa.FA_F32, "f16": fa.FA_F16, "bf16": fa.FA_BF16, "fp8_e4m3": fa.FA_FP8_E4M3}[w.dtype]
    return fa.fa_variant_name(code, w.d, w.causal, tile or 1)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def oracle_operands(w, x):
    """The exact values the kernel reads, as the oracle's inputs (E4M3: code x descale)."""
    import oracle
    if w.dtype == "fp8_e4m3":
        dq, dk, dv = x["descale"]
        return tuple(oracle.dequant_e4m3(t, s) for t, s in ((x["q"], dq), (x["k"], dk), (x["v"], dv)))
    return x["q"], x["k"], x["v"]


# parity bars of the forward: O max abs, O relative L2 over the compared
# rows, LSE max abs (None: not part of the bar for the dtype)
PARITY_BARS = {"f32": (1e-5, 1e-6, 1e-3), "f16": (2e-2, 5e-3, 1e-3), "bf16": (2e-2, 5e-3, 1e-3),
               "fp8_e4m3": (None, 5e-2, 1e-3)}


def one_thread_timings() -> dict:
    """The oracle on one thread: the 1x1x256x64 float32 workload whole, and
    one whole head (1024 rows) of the GPT-2-medium bf16 workload."""
    import oracle
    import torch
    from exact_attention_95_amd.inputs import WORKLOADS, head_normal, make_inputs
    prev = oracle.set_num_threads(1)
    out = {}
    try:
        w1 = WORKLOADS["single_head_f32_n256_d64"]
        x1 = make_inputs(w1)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.attention(x1["q"], x1["k"], x1["v"], w1.sm_scale, w1.causal)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 1.0:
                break
        out[w1.name] = {"gflops": round(w1.flops * reps / dt / 1e9, 3), "s_per_call": round(dt / reps, 5)}
        w2 = WORKLOADS["gpt2_medium_bf16_n1024_d64"]
        q, k, v = (torch.from_numpy(head_normal(w2.seed_id, t, 0, 0, w2.n_q, w2.d)).to(torch.bfloat16)
                   for t in range(3))
        t0 = time.perf_counter()
        oracle.attention(q, k, v, w2.sm_scale, w2.causal)
        dt = time.perf_counter() - t0
        f = 4.0 * w2.n_q * w2.n_kv * w2.d
        out[w2.name + "_one_head"] = {"gflops": round(f / dt / 1e9, 3), "s": round(dt, 3)}
    finally:
        oracle.set_num_threads(prev)
    return out


def cpu_baseline(w, x, o_gpu=None, lse_gpu=None, target_s: float = 25.0):
    """The fp64 oracle (as it stands) on the same workload: the whole workload
    when it takes about target_s seconds or less of host time, else a uniform
    row sample grown until one run takes about that long (the last run is
    reported).  Returns (baseline record, parity record): the oracle's rows
    are compared with the GPU's O and LSE (max abs, relative L2, LSE max
    abs over the compared rows)."""
    import oracle
    rng = np.random.default_rng([w.seed_id, 7])
    total = w.B * w.H * w.n_q

    def flops_of(rows):
        i = rows % w.n_q
        vis = np.minimum(i + 1, w.n_kv) if w.causal else np.full(rows.shape, w.n_kv)
        return float(np.sum(4.0 * vis * w.d))

    qo, ko, vo = oracle_operands(w, x)
    # grow the sample until it takes about target_s (the per-call fp64 conversion
    # of the touched heads is a fixed cost, so one calibration step undershoots)
    n = min(1024, total)
    while True:
        rows = np.arange(total) if n == total else np.sort(rng.choice(total, size=n, replace=False))
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attention(qo, ko, vo, w.sm_scale, w.causal, rows=rows)
        dt = time.perf_counter() - t0
        if dt >= 0.6 * target_s or n == total:
            break
        n = int(min(total, max(2 * n, n * target_s / max(dt, 1e-3))))
    f = flops_of(rows)
    whole = rows.size == total
    base = {
        "value": round(f / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": "%s of workload %s (%d of %d query rows); fp64 three-pass oracle, %.1f s, %.4g FLOP"
                  % ("the whole tensor" if whole else "a uniform row sample without replacement",
                     w.name, rows.size, total, dt, f),
        "one_thread": one_thread_timings(),
    }
    parity = None
    if o_gpu is not None:
        import torch
        sel = torch.from_numpy(rows).to(o_gpu.device)
        og = o_gpu.reshape(-1, w.d)[sel].double().cpu().numpy()
        diff = og - o_ref
        parity = {"rows": int(rows.size), "whole_tensor": bool(whole),
                  "max_abs": float(np.abs(diff).max()),
                  "rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(o_ref))}
        if lse_gpu is not None:
            lg = lse_gpu.reshape(-1)[sel].double().cpu().numpy()
            parity["lse_max_abs"] = float(np.abs(lg - lse_ref).max())
        bars = PARITY_BARS[w.dtype]
        parity["bars"] = {"max_abs": bars[0], "rel_l2": bars[1], "lse_max_abs": bars[2]}
        parity["within_bars"] = bool(
            np.isfinite(og).all() and (bars[0] is None or parity["max_abs"] <= bars[0])
            and parity["rel_l2"] <= bars[1] and parity.get("lse_max_abs", 0.0) <= bars[2])
    return base, parity


def cpu_baseline_bwd(w, x, dout, target_s: float = 15.0) -> dict:
    """The fp64 oracle's gradients (as they stand) on whole heads of the same
    workload: one head, then more until a run takes about target_s seconds.
    Counted with the metric's algorithmic FLOPs (10 N_q N_kv d per head,
    halved when causal)."""
    import oracle
    total = w.B * w.H
    n = 1
    while True:
        heads = list(range(n))
        q = np.stack([x["q"].reshape(total, w.n_q, w.d)[i].double().numpy() for i in heads])[:, None]
        k = np.stack([x["k"].reshape(total, w.n_kv, w.d)[i].double().numpy() for i in heads])[:, None]
        v = np.stack([x["v"].reshape(total, w.n_kv, w.d)[i].double().numpy() for i in heads])[:, None]
        g = np.stack([dout.reshape(total, w.n_q, w.d)[i].double().numpy() for i in heads])[:, None]
        t0 = time.perf_counter()
        oracle.backward(q, k, v, g, w.sm_scale, w.causal)
        dt = time.perf_counter() - t0
        if dt >= 0.6 * target_s or n == total:
            break
        n = int(min(total, max(n + 1, n * target_s / max(dt, 1e-3))))
    f = w.bwd_flops / total * n
    return {
        "value": round(f / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "%d of %d heads of workload %s (whole heads); fp64 oracle gradients, %.1f s, "
                  "%.4g FLOP counted as 10*N_q*N_kv*d per head" % (n, total, w.name, dt, f),
    }


def summarize_counters(workload: str, fetch_csv: str, write_csv: str, variant: str,
                       bwd: bool = False) -> dict:
    """HBM bytes per launch of the attention kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE, KiB per dispatch), each scaled by what the same
    counter reads for a plain 1 GiB device copy (hipMemcpy's copy kernel) run
    in the same process (bench.py --copy-calibration)."""
    import csv
    from exact_attention_95_amd.inputs import WORKLOADS

    def per_kernel(path, counter):
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    def factor_and_value(path, counter):
        rows = per_kernel(path, counter)
        copy = [v for k, vals in rows.items() if "copyBuffer" in k for v in vals]
        # per launch: the forward kernel, or the sum of the backward's three
        # kernels (each averaged over its dispatches)
        key = "bwd_" if bwd else "fwd"
        groups = [vals for k, vals in rows.items() if key in k and "fa" in k]
        if not copy or not groups:
            raise RuntimeError("missing copy or attention dispatches in %s" % path)
        copy_kib = sorted(copy)[len(copy) // 2]
        factor = (1 << 30) / (copy_kib * 1024.0)
        value = sum(sum(v) / len(v) for v in groups) * 1024.0
        return factor, value

    ff, fetch = factor_and_value(fetch_csv, "FETCH_SIZE")
    wf, write = factor_and_value(write_csv, "WRITE_SIZE")
    rec = {
        "workload": workload + ("_bwd" if bwd else ""),
        "kernel_source_digest": kernel_source_digest(WORKLOADS[workload].dtype, bwd),
        "variant": variant,
        "fetch_bytes_raw": fetch, "fetch_factor": ff,
        "write_bytes_raw": write, "write_factor": wf,
        "hbm_bytes_per_launch": round(fetch * ff + write * wf),
    }
    return rec


def launch_stats(step, stream, n: int, flush=None) -> dict:
    """Per-launch durations (ms) of n launches, each bracketed by HIP events on
    the launch stream; with flush, a device buffer is overwritten before every
    launch so that the launch starts with cold caches (L2 and the 256 MB
    Infinity Cache)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    with torch.cuda.stream(stream):
        for i, (a, b) in enumerate(evs):
            if flush is not None:
                flush.fill_(i & 0x7F)
            a.record(stream)
            step()
            b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return {"median": round(float(np.median(ms)), 4), "min": round(ms[0], 4),
            "max": round(ms[-1], 4), "launches": n}


# matrix-core FLOPs per clock and CU (the published peak / (256 CUs x 2.4 GHz))
MFMA_FLOP_PER_CLK_CU = {"bf16": 4096, "f16": 4096, "fp8_e4m3": 8192, "f32": 256}


def device_probe(dtype: str, stream) -> dict:
    """Rates measured on this device by the library's probe kernels: the
    sustained MFMA rate of the workload's input type, v_exp_f32 and fp32 FMA
    throughput, and the shader clock while each ran (cycle counter against
    the constant wall clock)."""
    import torch
    from exact_attention_95_amd import fa
    kind_of = {"bf16": fa.FA_PROBE_MFMA_BF16, "f16": fa.FA_PROBE_MFMA_F16,
               "fp8_e4m3": fa.FA_PROBE_MFMA_FP8, "f32": fa.FA_PROBE_MFMA_F32}
    khz = fa.fa_probe_wall_clock_khz()

    def run(kind, n_wg, iters):
        sink = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
        clocks = torch.zeros(n_wg * 8, dtype=torch.int64, device="cuda")
        for it in (max(1, iters // 16), iters):  # warm-up, then the timed launch
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            st = fa.fa_probe(kind, n_wg, it, sink.data_ptr(), clocks.data_ptr(), stream.cuda_stream)
            ev1.record(stream)
            if st != fa.FA_OK:
                raise fa.FaError(st)
            torch.cuda.synchronize()
        sec = ev0.elapsed_time(ev1) * 1e-3
        work = n_wg * 4 * iters * fa.fa_probe_work_per_iter(kind)
        c = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
        ghz = float(np.median(c[:, 0] / c[:, 1])) * khz * 1e-6 if khz > 0 else None
        return work / sec, ghz

    # 2 waves per SIMD for the MFMA loop, 8 for the VALU loops
    rate, ghz = run(kind_of[dtype], 512, {"fp8_e4m3": 32768, "f32": 32768}.get(dtype, 65536))
    exp_rate, exp_ghz = run(fa.FA_PROBE_EXP, 2048, 16384)
    fma_rate, fma_ghz = run(fa.FA_PROBE_FMA, 2048, 65536)
    per_clk = lambda r, g: round(r / (256 * g * 1e9), 2) if g else None
    return {
        "mfma_tflops": round(rate / 1e12, 1), "mfma_dtype": dtype,
        "clock_ghz_during_mfma": round(ghz, 3) if ghz else None,
        "mfma_flop_per_clk_cu": per_clk(rate, ghz),
        "mfma_flop_per_clk_cu_published": MFMA_FLOP_PER_CLK_CU[dtype],
        "exp_per_clk_cu": per_clk(exp_rate, exp_ghz), "clock_ghz_during_exp": exp_ghz and round(exp_ghz, 3),
        "fma_per_clk_cu": per_clk(fma_rate, fma_ghz), "clock_ghz_during_fma": fma_ghz and round(fma_ghz, 3),
    }


def hwmon_power_files():
    """(power1_input, power1_cap) sysfs paths of the first GPU that has them
    (values in microwatts), or (None, None)."""
    import glob
    for f in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input")):
        cap = f.replace("power1_input", "power1_cap")
        return f, (cap if os.path.exists(cap) else None)
    return None, None


def read_watts(path):
    try:
        with open(path) as f:
            return int(f.read().strip()) / 1e6
    except (OSError, ValueError, TypeError):
        return None


def sample_sclk_power():
    """(shader clock in MHz as rocm-smi reports it, package power in W from
    the GPU's hwmon sysfs file); None for a value that is not available."""
    import re
    import subprocess
    clk = None
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                             timeout=10).stdout
        for line in out.splitlines():
            if "sclk" in line:
                m = re.search(r"\((\d+)\s*Mhz\)", line, re.IGNORECASE)
                if m:
                    clk = int(m.group(1))
                    break
    except (OSError, subprocess.SubprocessError):
        pass
    return clk, read_watts(hwmon_power_files()[0])


def timed_with_clock(fn, stream, seconds: float) -> dict:
    """Runs fn back to back on `stream` for about `seconds` while a thread samples
    the shader clock and package power; returns ms per call (HIP events) and
    their medians."""
    import threading

    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    n = max(10, int(seconds * 1e3 / max(e0.elapsed_time(e1), 1e-3)))
    clocks, watts, done = [], [], threading.Event()

    def sampler():
        time.sleep(0.3)  # past the ramp at the start of the run
        while not done.is_set():
            c, w = sample_sclk_power()
            if c is None and w is None:
                return
            if c is not None:
                clocks.append(c)
            if w is not None:
                watts.append(w)
            time.sleep(0.1)

    th = threading.Thread(target=sampler)
    e0.record(stream)
    th.start()
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    done.set()
    th.join()
    return {"ms": round(e0.elapsed_time(e1) / n, 4), "calls": n,
            "sclk_mhz_median": float(np.median(clocks)) if clocks else None,
            "sclk_samples": len(clocks),
            "power_w_median": float(np.median(watts)) if watts else None}


def power_check(w, step, inputs, stream, flops: float, refresh=None, pass_name: str = "fwd",
                seconds: float = 2.0) -> dict:
    """The same launches on the workload's seeded inputs and on all-zero inputs
    (identical instruction stream, no data toggling), and hipBLASLt's
    8192^3 bf16 GEMM (torch.matmul) on N(0,1) and on all-zero operands, each
    run for about `seconds` with the shader clock and package power sampled.
    Tells a kernel limited by its instruction stream from one limited by the
    power draw of its data.  `inputs` are the tensors zeroed; `refresh`, if
    given, recomputes what the step reads besides them (the backward reads the
    forward's O and LSE) after they change."""
    import torch
    rec = {"workload": w.name, "pass": pass_name, "power_cap_w": read_watts(hwmon_power_files()[1])}
    with torch.cuda.stream(stream):
        rec["attention_seeded"] = timed_with_clock(step, stream, seconds)
        saved = [t.clone() for t in inputs]
        for t in inputs:
            t.zero_()
        if refresh:
            refresh()
        rec["attention_zeros"] = timed_with_clock(step, stream, seconds)
        for t, s in zip(inputs, saved):
            t.copy_(s)
        if refresh:
            refresh()
        del saved
        for r in (rec["attention_seeded"], rec["attention_zeros"]):
            r["tflops"] = round(flops / (r["ms"] * 1e-3) / 1e12, 1)
        m = 8192
        dev = inputs[0].device
        gen = torch.Generator(device=dev).manual_seed(0)
        a = torch.randn(m, m, device=dev, generator=gen).to(torch.bfloat16)
        b = torch.randn(m, m, device=dev, generator=gen).to(torch.bfloat16)
        c = torch.empty(m, m, device=dev, dtype=torch.bfloat16)
        rec["gemm8192_bf16_randn"] = timed_with_clock(lambda: torch.matmul(a, b, out=c), stream, seconds)
        a.zero_()
        b.zero_()
        rec["gemm8192_bf16_zeros"] = timed_with_clock(lambda: torch.matmul(a, b, out=c), stream, seconds)
        for key in ("gemm8192_bf16_randn", "gemm8192_bf16_zeros"):
            rec[key]["tflops"] = round(2 * m ** 3 / (rec[key]["ms"] * 1e-3) / 1e12, 1)
    torch.cuda.synchronize()
    rec["attention_over_gemm_seeded"] = round(
        rec["attention_seeded"]["tflops"] / rec["gemm8192_bf16_randn"]["tflops"], 4)
    return rec


def hbm_reference(dev, nbytes: int = 4 << 30, reps: int = 10) -> dict:
    """GB/s of the library's streaming-read probe (fa_probe_hbm_read, 8192
    workgroups), of torch's device copy (bytes read + written) and of a
    float32 sum over bf16 data (bytes read), each on `nbytes` of input."""
    import torch
    from exact_attention_95_amd import fa
    x = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).normal_()
    y = torch.empty_like(x)
    acc = torch.empty((), dtype=torch.float32, device=dev)

    def rate(fn, moved):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(moved / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)

    n_wg = 8192
    sink = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)

    def probe():
        st = fa.fa_probe_hbm_read(x.data_ptr(), nbytes, n_wg, sink.data_ptr(),
                                  torch.cuda.current_stream(dev).cuda_stream)
        if st != fa.FA_OK:
            raise fa.FaError(st)

    rec = {"bytes": nbytes,
           "read_probe_GBps": rate(probe, nbytes),
           "copy_GBps": rate(lambda: y.copy_(x), 2 * nbytes),
           "sum_read_GBps": rate(lambda: acc.copy_(x.sum(dtype=torch.float32)), nbytes)}
    del x, y
    return rec


def memory_report(names) -> list:
    """Device memory of fa_fwd (inputs, outputs and nothing else) against the
    analytic footprint of materialising S and P (N x N each, input dtype)."""
    import torch
    from exact_attention_95_amd import fa
    from exact_attention_95_amd.inputs import WORKLOADS, make_inputs
    out = []
    for name in names:
        w = WORKLOADS[name]
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        x = make_inputs(w)
        q, k, v = (x[n].to("cuda") for n in ("q", "k", "v"))
        del x
        o, lse = fa.fwd(q, k, v, scale=w.sm_scale, causal=w.causal)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        esize = q.element_size()
        tensors = (q.numel() + k.numel() + v.numel() + o.numel()) * esize + lse.numel() * 4
        s_and_p = 2 * w.B * w.H * w.n_q * w.n_kv * esize
        out.append({"workload": name, "device_bytes_peak": peak, "inputs_outputs_bytes": tensors,
                    "materialised_s_p_bytes": s_and_p,
                    "materialised_fits_288GB": bool(s_and_p + tensors < 288e9)})
        del q, k, v, o, lse
    return out


# Every other workload of the forward table, and the backward, timed after
# the headline's timed region (forward unless noted)
OTHER_WORKLOADS = [("single_head_f32_n256_d64", "fwd"), ("gpt2_medium_bf16_n1024_d64", "fwd"),
                   ("long_f16_causal_n4096_d64", "fwd"), ("long_f16_causal_n16384_d64", "fwd"),
                   ("long_f16_causal_n65536_d64", "fwd"), ("headline_bf16_n8192_d128", "fwd"),
                   ("headline_bf16_causal_n8192_d128", "fwd"), ("large_head_bf16_n16384_d256", "fwd"),
                   ("fp8_e4m3_n16384_d128", "fwd"), ("decode_bf16_b8_h32_nkv65536_d128", "splitkv"),
                   ("decode_e4m3_b8_h32_nkv65536_d128", "splitkv"),
                   ("headline_bf16_n8192_d128", "bwd"), ("large_head_bf16_n16384_d256", "bwd")]


def device_inputs(w, dev):
    """Seeded N(0,1) inputs of w's shape drawn on the device (torch's generator;
    fast for the large shapes), cast as make_inputs does: 16-bit by RNE, E4M3
    with per-tensor absmax scaling to 448, and w.boost on a fraction of Q's
    rows.  For timing only; parity runs on the oracle's inputs."""
    import torch
    from exact_attention_95_amd.inputs import DTYPES, E4M3_MAX
    g = torch.Generator(device=dev).manual_seed(1000 + w.seed_id)
    q = torch.randn((w.B, w.H, w.n_q, w.d), generator=g, device=dev)
    k = torch.randn((w.B, w.H, w.n_kv, w.d), generator=g, device=dev)
    v = torch.randn((w.B, w.H, w.n_kv, w.d), generator=g, device=dev)
    if w.boost_frac:
        rows = torch.randperm(w.B * w.H * w.n_q, generator=g, device=dev)[:int(w.boost_frac * w.B * w.H * w.n_q)]
        q.view(-1, w.d)[rows] *= w.boost
    if w.dtype == "fp8_e4m3":
        out, desc = [], []
        for t in (q, k, v):
            sc = E4M3_MAX / float(t.abs().max())
            out.append((t * sc).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn))
            desc.append(1.0 / sc)
        return out[0], out[1], out[2], tuple(desc)
    dt = DTYPES[w.dtype]
    return q.to(dt), k.to(dt), v.to(dt), (1.0, 1.0, 1.0)


def other_workloads(dev, seconds: float = 0.6) -> list:
    """Each workload of OTHER_WORKLOADS in its default launch configuration,
    run back to back for about `seconds` on device-drawn inputs with the
    shader clock and package power sampled: ms per call (HIP events),
    TFLOP/s (decode: GB/s of algorithmic bytes), fraction of the dtype's
    peak, and joules per TFLOP."""
    import torch
    from exact_attention_95_amd import fa
    from exact_attention_95_amd.inputs import WORKLOADS
    out = []
    for name, kind in OTHER_WORKLOADS:
        w = WORKLOADS[name]
        q, k, v, desc = device_inputs(w, dev)
        od = torch.bfloat16 if w.dtype == "fp8_e4m3" else q.dtype
        o = torch.empty(q.shape, dtype=od, device=dev)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        stream = torch.cuda.Stream(device=dev)
        args = fa.make_args(q, k, v, o, lse, w.sm_scale, w.causal, desc, stream.cuda_stream, 0)
        keep = []
        if kind == "splitkv":
            ws = torch.empty(max(fa.fa_splitkv_workspace_bytes(args, 0), 256), dtype=torch.uint8, device=dev)
            keep.append(ws)
            fn = lambda: fa.fa_fwd_splitkv(args, 0, ws.data_ptr(), ws.numel())
        elif kind == "bwd":
            with torch.cuda.stream(stream):
                fa.fa_fwd_ex(args)
            do = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(4), device=dev).to(q.dtype)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            bargs = fa.make_bwd_args(q, k, v, o, lse, do, dq, dk, dv, w.sm_scale, w.causal, stream.cuda_stream)
            ws = torch.empty(max(fa.fa_bwd_workspace_bytes(bargs), 256), dtype=torch.uint8, device=dev)
            keep += [do, dq, dk, dv, ws]
            fn = lambda: fa.fa_bwd(bargs, ws.data_ptr(), ws.numel())
        else:
            fn = lambda: fa.fa_fwd_ex(args)
        st = fn()
        if st != fa.FA_OK:
            raise fa.FaError(st)
        r = timed_with_clock(fn, stream, seconds)
        flops = w.bwd_flops if kind == "bwd" else w.flops
        rec = {"workload": name, "pass": kind, "variant": variant_label(name, bwd=(kind == "bwd")),
               "ms": r["ms"], "calls": r["calls"], "sclk_mhz_median": r["sclk_mhz_median"],
               "power_w_median": r["power_w_median"]}
        if kind == "splitkv":
            gbs = algorithmic_bytes(w) / (r["ms"] * 1e-3) / 1e9
            rec.update(GBps=round(gbs, 1), frac=round(gbs / PEAK_HBM_GBS, 4), bound="hbm")
        else:
            tf = flops / (r["ms"] * 1e-3) / 1e12
            rec.update(tflops=round(tf, 1), frac=round(tf / PEAK_TFLOPS[w.dtype], 4), bound="mfma")
            if r["power_w_median"]:
                rec["joules_per_tflop"] = round(r["power_w_median"] * r["ms"] * 1e-3 / (flops / 1e12), 4)
        out.append(rec)
        del q, k, v, o, lse, keep, args
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1,
                    help="number of GPUs; only 1 is supported (the path runs on one GPU)")
    ap.add_argument("--steps", type=int, default=50, help="timed steps (one call over the whole batch each)")
    ap.add_argument("--warmup", type=int, default=10, help="untimed steps before the timed region")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="workload name (default: %(default)s); see exact_attention_95_amd/inputs.py")
    ap.add_argument("--tile", type=int, default=0, help="fa_fwd_args.tile_override")
    ap.add_argument("--splitkv", type=int, default=None,
                    help="use the split-KV entry point with this many chunks (0: library "
                         "choice, -1: off); default: on for workloads with at most 16 query rows")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (fa_bwd: dQ, dK, dV) instead of the forward")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout probability (Philox mask, seed 1, offset 0) for the forward "
                         "and --bwd runs")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (and the parity check it carries)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc "
                         "counter_collection.csv files and exit")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-launch (warm and cold-cache) timings and the device "
                         "probes that follow the timed region (for profiler runs)")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="time every compiled variant (tile shape) for the workload's dtype, "
                         "head dim and mask, one JSON line each, and exit")
    ap.add_argument("--power-check", action="store_true",
                    help="time the forward on the seeded inputs and on all-zero inputs, and "
                         "hipBLASLt's 8192^3 bf16 GEMM on N(0,1) and on zero operands, with the "
                         "shader clock sampled, print one JSON line and exit")
    ap.add_argument("--other-workloads", type=int, default=1,
                    help="1 (default): after the timed region, also time every other forward "
                         "workload, the split-KV decode and the backward (about 1 s each) and add "
                         "them to the JSON line; 0: skip")
    ap.add_argument("--memory-report", action="store_true",
                    help="print device memory of the long causal fp16 workloads vs a "
                         "materialised N x N baseline and exit")
    args = ap.parse_args(argv)

    if args.summarize_counters:
        rec = summarize_counters(args.workload, *args.summarize_counters,
                                 variant=variant_label(args.workload, args.tile, args.splitkv, args.bwd),
                                 bwd=args.bwd)
        path = os.path.join(TRAFFIC_DIR, "traffic_%s.json" % rec["workload"])
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the multi-GPU split (heads across GPUs, "
              "no exchange) is not built.", file=sys.stderr)
        return 2

    import torch
    from exact_attention_95_amd import fa
    from exact_attention_95_amd.inputs import WORKLOADS, make_dout, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.memory_report:
        for rec in memory_report(["long_f16_causal_n4096_d64", "long_f16_causal_n16384_d64",
                                  "long_f16_causal_n65536_d64"]):
            print(json.dumps(rec), flush=True)
        return 0
    w = WORKLOADS[args.workload]
    x = make_inputs(w)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    out_dtype = torch.bfloat16 if w.dtype == "fp8_e4m3" else q.dtype
    o = torch.empty(q.shape, dtype=out_dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)  # default priority
    fargs = fa.make_args(q, k, v, o, lse, w.sm_scale, w.causal, x["descale"],
                         stream.cuda_stream, args.tile, (args.dropout, 1, 0))
    st = fa.fa_validate(fargs)
    if st != fa.FA_OK:
        raise fa.FaError(st)
    splitkv = args.splitkv if args.splitkv is not None else (0 if w.n_q <= 16 else None)
    if splitkv is not None and splitkv < 0:  # -1: force the single-pass entry point
        splitkv = None
    if splitkv is not None:
        need = fa.fa_splitkv_workspace_bytes(fargs, splitkv)
        if need < 0:
            raise fa.FaError(fa.FA_ERR_VARIANT)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

        def step():
            s = fa.fa_fwd_splitkv(fargs, splitkv, workspace.data_ptr(), workspace.numel())
            if s != fa.FA_OK:
                raise fa.FaError(s)
    else:
        def step():
            s = fa.fa_fwd_ex(fargs)
            if s != fa.FA_OK:
                raise fa.FaError(s)
    check = o
    if args.bwd:
        if w.dtype not in ("bf16", "f16") or w.d not in (64, 128, 256):
            print("the backward covers bf16/fp16 with d in {64, 128, 256}", file=sys.stderr)
            return 2
        # the forward's O and LSE, then the timed step is one fa_bwd call
        fwd_step = step
        step()
        do = make_dout(w).to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bargs = fa.make_bwd_args(q, k, v, o, lse, do, dq, dk, dv, w.sm_scale, w.causal,
                                 stream.cuda_stream, (args.dropout, 1, 0))
        bneed = fa.fa_bwd_workspace_bytes(bargs)
        if bneed < 0:
            raise fa.FaError(fa.fa_bwd_validate(bargs))
        bws = torch.empty(max(bneed, 256), dtype=torch.uint8, device=dev)
        check = dk

        def step():
            s = fa.fa_bwd(bargs, bws.data_ptr(), bws.numel())
            if s != fa.FA_OK:
                raise fa.FaError(s)

    if args.tile_sweep:
        if args.bwd or splitkv is not None:
            print("--tile-sweep covers the single-pass forward", file=sys.stderr)
            return 2
        # each variant runs back to back for about a second, long enough for
        # the board's power management to settle (short bursts run at a
        # higher clock); two passes, so drift of the board shows
        n_var = fa.fa_num_variants(fargs.dtype, w.d, w.causal)
        for rep in range(2):
            for tile in range(1, n_var + 1):
                fargs.tile_override = tile
                r = timed_with_clock(step, stream, 1.0)
                print(json.dumps({"workload": w.name, "pass": rep, "tile_override": tile,
                                  "variant": fa.fa_variant_name(fargs.dtype, w.d, w.causal, tile),
                                  "default": tile == 1, **r,
                                  "tflops": round(w.flops / (r["ms"] * 1e-3) / 1e12, 1)}), flush=True)
        return 0

    if args.power_check:
        if splitkv is not None:
            print("--power-check covers the single-pass forward and the backward", file=sys.stderr)
            return 2
        if args.bwd:
            rec = power_check(w, step, (q, k, v, do), stream, w.bwd_flops, refresh=fwd_step,
                              pass_name="bwd")
        else:
            rec = power_check(w, step, (q, k, v), stream, w.flops)
        print(json.dumps(rec), flush=True)
        return 0

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    if not bool(torch.isfinite(check.float()).all()):
        print("non-finite output", file=sys.stderr)
        return 1

    extras = {}
    if not args.no_extras:
        # per-launch spread, warm and with cold caches (512 MB written between
        # launches), then the device's own rates; all after the timed region
        extras["launch_ms"] = {"warm": launch_stats(step, stream, args.steps)}
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        extras["launch_ms"]["cold"] = launch_stats(step, stream, args.steps, flush)
        extras["launch_ms"]["cold"]["flush_bytes"] = flush.numel()
        del flush
        extras["device"] = device_probe(w.dtype, stream)
        # shader clock and package power while the same step runs back to back
        # for about a second (random data: the board's power cap sets the clock)
        under = timed_with_clock(step, stream, 1.0)
        flops_step = w.bwd_flops if args.bwd else w.flops
        extras["device"]["under_kernel"] = {
            "ms": under["ms"], "sclk_mhz_median": under["sclk_mhz_median"],
            "power_w_median": under["power_w_median"],
            "power_cap_w": read_watts(hwmon_power_files()[1]),
            # energy per unit of work under the cap: power x time / FLOPs
            "joules_per_tflop": (round(under["power_w_median"] * under["ms"] * 1e-3 / (flops_step / 1e12), 4)
                                 if under["power_w_median"] else None)}
        if (args.other_workloads and w.name == DEFAULT_WORKLOAD and not args.bwd and splitkv is None
                and args.dropout == 0.0 and args.tile == 0):
            # the forward table's other workloads and the backward, timed after
            # the headline's timed region on device-drawn inputs
            extras["other_workloads"] = other_workloads(dev)

    if args.copy_calibration:
        # a plain device-to-device copy of exactly 1 GiB (hipMemcpy's copy kernel)
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    flops = w.bwd_flops if args.bwd else w.flops
    value = flops * args.steps / wall / 1e12
    nbytes = algorithmic_bytes_bwd(w) if args.bwd else algorithmic_bytes(w)
    # the bound of the dominant kernel: HBM when the arithmetic intensity is
    # below the dtype's ridge point, else the matrix cores
    hbm_bound = flops / nbytes < PEAK_TFLOPS[w.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:
        achieved, peak, unit = nbytes / (kernel_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = flops / (kernel_ms * 1e-3) / 1e12, PEAK_TFLOPS[w.dtype], "TFLOP/s"
    rec = {
        "metric": BWD_METRIC if args.bwd else METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N_q": w.n_q, "N_kv": w.n_kv,
                   "d": w.d, "causal": w.causal, "dtype": w.dtype,
                   "dropout_p": args.dropout,
                   "variant": variant_label(w.name, args.tile, args.splitkv, args.bwd),
                   "flops_per_step": flops, "algorithmic_bytes_per_step": nbytes},
        # HBM bytes the two traffic models of the pages give for this launch,
        # beside the measured traffic (fwd only)
        "traffic_models": None if args.bwd or splitkv is not None else {
            "materialised_s_and_p": materialised_bytes(w),
            "tiled_without_cache_reuse": fa_bytes_without_l2(w, variant_rows(
                fa.fa_variant_name(fargs.dtype, w.d, w.causal, args.tile or 1)))},
        "roofline": {"bound": "hbm" if hbm_bound else "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": stored_traffic(w.name, w.dtype,
                                               variant_label(w.name, args.tile, args.splitkv, args.bwd),
                                               args.bwd),
                     "kernel_ms": round(kernel_ms, 4)},
    }
    if extras and hbm_bound:
        # what plain streaming reaches on this HBM, for scale: the library's
        # read probe, torch's device copy (read + write) and a float32 sum
        # (read), 4 GiB each
        extras["hbm_reference"] = hbm_reference(dev)
    if extras:
        rec.update(extras)
        if hbm_bound:
            # the kernel's rate against the read rate measured on this device
            rec["roofline"]["frac_of_measured_peak"] = round(
                achieved / extras["hbm_reference"]["read_probe_GBps"], 4)
        else:
            # the kernel's rate against the MFMA rate measured on this device
            rec["roofline"]["frac_of_measured_peak"] = round(
                achieved / extras["device"]["mfma_tflops"], 4)
    if not args.no_cpu_baseline and args.dropout == 0.0:
        if args.bwd:
            rec["cpu_baseline"] = cpu_baseline_bwd(w, x, do.cpu())
        else:
            rec["cpu_baseline"], rec["parity"] = cpu_baseline(w, x, o, lse)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
