#!/usr/bin/env python3
"""MoE layer forward throughput on one MI355X.

One step = one full MoE layer forward (router, dispatch, grouped SwiGLU expert
FFN, combine) over one batch of T tokens, through libmoe's C ABI, with inputs
and weights already resident in HBM. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-all-configs]

The default workload is the largest configuration, the DeepSeek-V3-shaped
prefill layer (4096 tokens, 256 fp8 experts + 1 shared). The dominant kernel
(the routed gate/up grouped GEMM with fused SwiGLU, which streams two thirds of
the touched expert weights) is timed with HIP events recorded by libmoe on its
own stream around that kernel, in every timed step. Per-step latency (p50,
p95) and per-stage times come from separate passes. After the headline, every
other configuration is timed in the same run (key "configs").
"""
from __future__ import annotations

import argparse
import dataclasses
import csv
import glob
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 1 GPU + % HBM peak (decode) / % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
DECODE_WORKLOADS = {"toy_fp32", "mixtral_decode", "qwen3_decode", "dsv3_decode", "dsv3_decode_bf16_shared",
                    "mixtral_decode_mxfp4", "qwen3_decode_mxfp4"}
PROFILE_DIR = os.path.join(ROOT, "profiles")
# sources of the gate/up kernel each path launches (the traffic record is
# void once any of them changes)
KERNEL_SOURCES = {"stream": ("stream_gemm.hip", "common.h"),
                  "tiled": ("tiled_gemm_kernel.h", "tiled_gemm_bm128.hip", "tiled_gemm_bm256.hip", "common.h"),
                  "a8": ("tiled_a8.hip", "tiled_gemm_kernel.h", "common.h"),
                  "persist": ("tiled_persist.hip", "tiled_gemm_kernel.h", "common.h")}


def kernel_family(name: str) -> str:
    """Source family of a gate/up kernel's (demangled) name."""
    if "stream_gemm" in name:
        return "stream"
    return "a8" if "tiled_a8" in name else ("persist" if "tiled_persist" in name else "tiled")


def kernel_source_hash(path: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[path]:
        p = os.path.join(ROOT, "mixture_experts_layer_count_amd", "csrc", name)
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from a committed PMC summary, or None
    when none exists or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_hash") != kernel_source_hash(kernel_family(rec.get("kernel", ""))):
        return None
    return rec.get("hbm_bytes_per_launch")


def weight_bytes(cfg, dt=None) -> float:
    """Bytes per weight value, scales excluded (MXFP4: two values a byte)."""
    return {"f32": 4.0, "bf16": 2.0, "fp8": 1.0, "mxfp4": 0.5}[dt or cfg.w]


def scale_bytes(cfg, K: int, N: int, dt=None) -> float:
    """Scale bytes of one [K, N] weight matrix: fp32 per 128x128 block (fp8),
    one E8M0 byte per 32 K rows of a column (MXFP4), none otherwise."""
    dt = dt or cfg.w
    if dt == "fp8":
        return (K // 128) * (N // 128) * 4.0
    if dt == "mxfp4":
        return (K // 32) * N * 1.0
    return 0.0


def gate_bytes(cfg) -> float:
    """Bytes of the gate matrix (fp32, or the activation dtype)."""
    return cfg.H * cfg.E * (4.0 if "f32" in (cfg.wg, cfg.act) else 2.0)


def shared_bytes(cfg) -> float:
    """Weight (and fp8 block-scale) bytes of the shared expert."""
    if cfg.Fs == 0:
        return 0.0
    b = 3 * cfg.H * cfg.Fs * weight_bytes(cfg, cfg.shared_w)
    b += 2 * scale_bytes(cfg, cfg.H, cfg.Fs, cfg.shared_w) + scale_bytes(cfg, cfg.Fs, cfg.H, cfg.shared_w)
    return b


def cpu_baseline(cfg, d, k: int) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the same layer."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info

    n = cfg.T if cfg.T <= 64 and cfg.E <= 16 else (16 if cfg.E <= 16 else 4)
    tokens = np.arange(min(n, cfg.T))
    # host copies of the sample's inputs: its token rows, the gate, the shared
    # expert, and only the experts the sample's tokens choose (the whole
    # DeepSeek-shaped layer is 11 GB)
    small = {key: (v.cpu() if hasattr(v, "cpu") else v) for key, v in d.items()
             if key not in ("W1", "W3", "W2", "S1", "S3", "S2")}
    _, idx, _ = oracle.route(oracle.to_f64(small["X"][: len(tokens)]), small["Wg"], small.get("gate_bias"), k)
    chosen = sorted(set(int(e) for e in np.unique(idx)))
    host = dict(small)
    for key in ("W1", "W3", "W2", "S1", "S3", "S2"):
        if d.get(key) is not None:
            host[key] = _HostExperts(d[key], chosen)
    L = oracle.Layer(host, k)
    # repeat the sample until about 10 s of CPU work have been timed
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.forward_tokens(L, tokens)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or passes >= 64:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {"value": passes * len(tokens) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(tokens)} of {cfg.T} tokens x {passes} passes, full fp64 layer forward (route over "
                      f"all E, SwiGLU of each chosen expert, combine); {dt:.1f} s on {cpu_model()}"}


class _HostExperts:
    """Host copies of some experts of a stacked [E, ...] device tensor,
    indexed by expert like the tensor itself."""

    def __init__(self, t, experts):
        self.shape = tuple(t.shape)
        self.dtype = t.dtype
        self._rows = {e: t[e].cpu() for e in experts}

    def __getitem__(self, e):
        return self._rows[int(e)]


def cpu_model() -> str:
    """The host processor's model name (from /proc/cpuinfo on Linux)."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "host"


GATE_UP_KERNEL = re.compile(r"(stream|tiled)_gemm_kernel<[^,]+, true|tiled_a8_kernel<true")
# the routed down projection: the plain tiled kernel of 256- or 160-row tiles,
# or its persistent form (the 128-row fp32 form is the router's gate GEMM)
DOWN_KERNEL = re.compile(r"tiled_gemm_kernel<[^,]+, false, 256|tiled_a8_kernel<false|tiled_persist_kernel")


def _pmc_means(run_dir: str, counter: str) -> dict:
    """Mean per-dispatch value of one counter, per kernel name, from a
    rocprofv3 `--pmc ... -f csv` output directory."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per_dispatch = {}
    for f in files:
        with open(f, newline="", encoding="utf-8") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (f, r["Dispatch_Id"], r["Kernel_Name"])
                per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    by_kernel = {}
    for (_, _, name), v in per_dispatch.items():
        by_kernel.setdefault(name, []).append(v)
    return {name: (sum(v) / len(v), len(v)) for name, v in by_kernel.items()}


def record_traffic(args) -> int:
    """Turn four rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE of the
    workload and of the copy calibration) into the committed per-launch HBM
    traffic record of the gate/up kernel."""
    fetch, write = _pmc_means(args.pmc_fetch, "FETCH_SIZE"), _pmc_means(args.pmc_write, "WRITE_SIZE")
    cal_f, cal_w = _pmc_means(args.calib_fetch, "FETCH_SIZE"), _pmc_means(args.calib_write, "WRITE_SIZE")
    nbytes = COPY_CALIBRATION_BYTES
    # the copy is the calibration run's kernel that reads the most; every
    # kernel of that run (fill, copy) writes the whole buffer
    f_fetch = nbytes / (max(v for v, _ in cal_f.values()) * 1024.0)
    f_write = nbytes / (max(v for v, _ in cal_w.values()) * 1024.0)
    which = getattr(args, "pmc_kernel", "gate_up")
    pattern = GATE_UP_KERNEL if which == "gate_up" else DOWN_KERNEL
    names = [n for n in fetch if pattern.search(n)]
    if len(names) != 1:
        raise SystemExit(f"expected one {which} kernel, found {names}")
    name = names[0]
    fk, nf = fetch[name]
    wk, nw = write[name]
    rec = {
        "workload": args.workload, "kernel": name,
        "kernel_source_hash": kernel_source_hash(kernel_family(name)),
        "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
        "dispatches": [nf, nw], "calibration_bytes": nbytes,
        "fetch_scale": round(f_fetch, 4), "write_scale": round(f_write, 4),
        "hbm_bytes_per_launch": round(fk * 1024.0 * f_fetch + wk * 1024.0 * f_write),
        "commands": args.commands,
    }
    stem = "gate_up_swiglu" if which == "gate_up" else "down"
    out = os.path.join(PROFILE_DIR, f"{stem}_{args.workload}_pmc.json")
    with open(out, "w", encoding="utf-8") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    with open(out[:-5] + ".md", "w", encoding="utf-8") as fh:
        fh.write(f"# HBM traffic of the {'gate/up SwiGLU' if which == 'gate_up' else 'down projection'} kernel: "
                 f"{args.workload}\n\n"
                 f"Kernel: `{name}` (sources hash {rec['kernel_source_hash']}).\n\n"
                 "| counter | KiB per dispatch | dispatches | scale | bytes per launch |\n|---|---:|---:|---:|---:|\n"
                 f"| FETCH_SIZE | {fk:.1f} | {nf} | {f_fetch:.4f} | {fk * 1024 * f_fetch:.4g} |\n"
                 f"| WRITE_SIZE | {wk:.1f} | {nw} | {f_write:.4f} | {wk * 1024 * f_write:.4g} |\n\n"
                 f"HBM bytes per launch: {rec['hbm_bytes_per_launch']:.4g}. The scales are what a {nbytes >> 20} MiB "
                 "device-to-device copy reads and writes, divided by what these counters report for it (its blit "
                 "kernel's FETCH_SIZE reports half the bytes read).\n\nCommands, from the repository root R:\n\n```\n"
                 + "\n".join(args.commands) + "\n```\n")
    print(json.dumps(rec))
    return 0


def summarize_trace(args) -> int:
    """Markdown table of libmoe's kernels from a rocprofv3 `--kernel-trace
    --stats -f csv` output directory (torch's own kernels left out)."""
    files = glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {args.summarize_trace}")
    rows = []
    with open(files[0], newline="", encoding="utf-8") as fh:
        for r in csv.DictReader(fh):
            name = r["Name"]
            if "moe::" not in name:
                continue
            name = re.sub(r"\(moe::GemmProblem, int\)|\((int|float|long|unsigned|short|moe::|const|uint4).*$", "",
                          name.replace("moe::(anonymous namespace)::", "")).strip()
            rows.append((name, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e3,
                         float(r["Percentage"])))
    print(f"# rocprofv3 kernel trace: {args.workload}\n")
    print("Commands, from the repository root R:\n\n```\n" + "\n".join(args.commands) + "\n```\n")
    print("| kernel | calls | avg (us) | total (us) | % of GPU time |\n|---|---:|---:|---:|---:|")
    for name, calls, avg, tot, pct in rows:
        print(f"| `{name}` | {calls} | {avg:.2f} | {tot:.1f} | {pct:.1f} |")
    print("\nKernels of torch (input generation, copies) are left out; the percentages are of all GPU time.")
    return 0


def summarize_counter(args) -> int:
    """Markdown table of one rocprofv3 counter (a derived one such as
    MfmaUtil, or a raw one) per libmoe GEMM kernel: its mean per dispatch,
    from a `--pmc <counter> -f csv` output directory."""
    means = _pmc_means(args.summarize_counter, args.counter)
    rows = [(re.sub(r"\(moe::GemmProblem.*$", "", n.replace("(anonymous namespace)::", "")).strip(), v, c)
            for n, (v, c) in means.items() if "_gemm_kernel" in n or "tiled_a8" in n or "tiled_persist" in n]
    if not rows:
        raise SystemExit(f"no GEMM kernel rows for {args.counter} under {args.summarize_counter}")
    print(f"# {args.counter} of the expert GEMM kernels: {args.workload}\n")
    print("Commands, from the repository root R:\n\n```\n" + "\n".join(args.commands) + "\n```\n")
    print(f"| kernel | dispatches | {args.counter} (mean per dispatch) |\n|---|---:|---:|")
    for name, v, c in sorted(rows):
        print(f"| `{name}` | {c} | {v:.2f} |")
    if args.counter == "MfmaUtil":
        print("\nMfmaUtil is rocprofv3's derived counter: the summed SQ_VALU_MFMA_BUSY_CYCLES over "
              "GRBM_GUI_ACTIVE times the SIMD count, in percent (matrix-core busy cycles, whatever the "
              "clock).")
    return 0


SWEEP_T = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192]


def t_sweep(args) -> int:
    """Token-count sweep of one model shape: the same layer (weights drawn
    once at the largest T) at T = 1 .. 8192 tokens, each row-streaming (gemv)
    and tiled path timed, plus the path AUTO takes. Reports ms per layer,
    tokens/s, the experts the batch touches and their weight bytes' share of
    the HBM peak (decode view) and the FFN flops' share of the dtype's MFMA
    peak (prefill view)."""
    import torch
    import mixture_experts_layer_count_amd as moe
    from synth import get_config, make_layer

    base = get_config(args.sweep)
    Ts = [t for t in SWEEP_T if t <= args.sweep_max_t]
    cfg = dataclasses.replace(base, name=f"{base.name}_sweep", T=max(Ts))
    d = make_layer(cfg, device="cuda")
    paths = ["gemv", "tiled"] + (["tiled_a8"] if cfg.w == "fp8" else [])
    layers = {p: moe.MoELayer(d, cfg.k, path=p) for p in paths + ["auto"]}
    wb = weight_bytes(cfg)
    rows = []
    for T in Ts:
        X = d["X"][:T].contiguous()
        Y = torch.empty_like(X)
        _, _, _, _, counts = layers["auto"].forward(X, Y, aux=True)
        torch.cuda.synchronize()
        touched = int((counts > 0).sum().item())
        w_bytes = touched * 3 * cfg.H * cfg.F * wb + shared_bytes(cfg) + gate_bytes(cfg)
        flops = 6.0 * T * cfg.k * cfg.H * cfg.F + 6.0 * T * cfg.H * cfg.Fs
        rec = {"T": T, "touched_experts": touched}
        steps = max(3, min(args.steps, int(2e4 // max(T, 1)) or 3))
        for name in paths + ["auto"]:
            layer = layers[name]
            for _ in range(2):
                layer.forward(X, Y)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                layer.forward(X, Y)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / steps
            # AUTO takes the tiled form from 15 rows per expert (W8A8 for fp8)
            a8 = name == "tiled_a8" or (name == "auto" and cfg.w == "fp8" and T * cfg.k >= 15 * cfg.E)
            rec[name] = {"ms": round(ms, 4), "tokens_per_s": round(T / ms * 1e3, 1),
                         "hbm_frac": round(w_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                         "mfma_frac": round(flops / (ms * 1e-3) /
                                            (MFMA_PEAK_TFLOPS["fp8" if a8 else "bf16"] * 1e12), 4)}
        best = min(paths, key=lambda n: rec[n]["ms"])
        rec["fastest"] = best
        rows.append(rec)
        print(json.dumps(rec), flush=True)
    print(f"\n| T | touched experts | " + " | ".join(f"{p} ms" for p in paths) +
          " | auto ms | fastest | auto tokens/s | auto HBM frac | auto MFMA frac |")
    print("|" + "---:|" * (len(paths) + 3) + "---|---:|---:|---:|")
    for r in rows:
        a = r["auto"]
        print(f"| {r['T']} | {r['touched_experts']} | " + " | ".join(f"{r[p]['ms']:.4f}" for p in paths) +
              f" | {a['ms']:.4f} | {r['fastest']} | {a['tokens_per_s']:.0f} | {a['hbm_frac']:.3f} | "
              f"{a['mfma_frac']:.3f} |")
    return 0


COPY_CALIBRATION_BYTES = 1 << 30


def copy_calibration(nbytes: int = COPY_CALIBRATION_BYTES) -> None:
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes}))


# HBM-graded workloads: decode batches (weights streamed for few rows) and the
# DeepSeek-shaped fp8 prefill, whose layer arithmetic intensity (about 287
# flop per byte) lies below the fp8 ridge, so HBM bounds it
HBM_GRADED = DECODE_WORKLOADS | {"dsv3_prefill", "dsv3_prefill_bf16_shared"}
# every configuration of the layer, timed beside the headline in one run
ALL_CONFIGS = ["toy_fp32", "mixtral_decode", "mixtral_prefill", "qwen3_decode", "qwen3_prefill",
               "dsv3_decode", "dsv3_prefill"]
EV_START, EV_SCHED, EV_GATE_UP, EV_COMBINE = 0, 3, 4, 8


def percentile(xs, q: float) -> float:
    """Linear-interpolated q-quantile (0 <= q <= 1) of a non-empty sample."""
    s = sorted(xs)
    pos = q * (len(s) - 1)
    lo = int(pos)
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (pos - lo)


def uses_a8(cfg, path: str) -> bool:
    """The W8A8 tiled kernels run (fp8 weights at prefill sizes under AUTO)."""
    if cfg.w != "fp8":
        return False
    return path == "tiled_a8" or (path == "auto" and cfg.T * cfg.k >= 15 * cfg.E)


def gate_up_work(cfg, touched: int, a8: bool):
    """Algorithmic bytes and flops of one routed gate/up launch (with the
    shared expert when it is a group of the same launch)."""
    wb = weight_bytes(cfg)
    ab = 4.0 if cfg.act == "f32" else 2.0
    xb = 1.0 if a8 else ab  # W8A8 reads E4M3 token rows and writes E4M3 h
    w = touched * 2 * (cfg.H * cfg.F * wb + scale_bytes(cfg, cfg.H, cfg.F))
    rows = cfg.T * cfg.k
    if cfg.Fs > 0 and cfg.Fs == cfg.F and cfg.shared_w == cfg.w:
        w += 2 * (cfg.H * cfg.Fs * wb + scale_bytes(cfg, cfg.H, cfg.Fs))
        rows += cfg.T
    act = cfg.T * cfg.H * xb + rows * cfg.F * xb
    if a8:  # per-row 128-column fp32 scales of the token rows and of h
        act += 4.0 * (cfg.T * cfg.H / 128 + rows * cfg.F / 128)
    return w + act, 4.0 * rows * cfg.H * cfg.F


def measure(cfg, path: str, steps: int, warmup: int, workload: str) -> dict:
    """Time `steps` layer forwards (after `warmup`) of one workload, with the
    gate/up kernel bracketed by HIP events in every timed step; then per-step
    latency and per-stage times in separate passes."""
    import torch
    import mixture_experts_layer_count_amd as moe
    from mixture_experts_layer_count_amd._lib import MOE_N_EVENTS
    from synth import make_layer

    d = make_layer(cfg, device="cuda")
    layer = moe.MoELayer(d, cfg.k, path=path)
    X = d["X"]
    Y = torch.empty_like(X)
    _, _, _, _, counts = layer.forward(X, Y, aux=True)
    torch.cuda.synchronize()
    touched = int((counts > 0).sum().item())

    evs = [moe.StageEvents(want=[EV_SCHED, EV_GATE_UP]) for _ in range(steps)]
    for _ in range(warmup):
        layer.forward(X, Y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        layer.forward(X, Y, events=evs[i].handles)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / steps
    gate_up_ms = statistics.fmean(e.elapsed_ms(EV_SCHED, EV_GATE_UP) for e in evs)

    # latency distribution: one marker pair around each whole forward
    n_lat = max(20, steps)
    lat_ev = [moe.StageEvents(want=[EV_START, EV_COMBINE]) for _ in range(n_lat)]
    for e in lat_ev:
        layer.forward(X, Y, events=e.handles)
    torch.cuda.synchronize()
    lat = [e.elapsed_ms(EV_START, EV_COMBINE) for e in lat_ev]
    # per-stage times: every marker recorded (each costs a few microseconds)
    stage_runs = []
    for _ in range(max(10, min(steps, 20))):
        ev = moe.StageEvents()
        layer.forward(X, Y, events=ev.handles)
        stage_runs.append([ev.elapsed_ms(i, i + 1) for i in range(MOE_N_EVENTS - 1)])
    torch.cuda.synchronize()
    stages = {name: {"p50": round(percentile([r[i] for r in stage_runs], 0.5), 4),
                     "p95": round(percentile([r[i] for r in stage_runs], 0.95), 4)}
              for i, name in enumerate(moe.STAGES)}

    a8 = uses_a8(cfg, path)
    gu_bytes, gu_flops = gate_up_work(cfg, touched, a8)
    mfma_dt = "f32" if cfg.w == "f32" else ("fp8" if a8 else "bf16")
    mfma_peak = MFMA_PEAK_TFLOPS[mfma_dt]
    gb_s = gu_bytes / (gate_up_ms * 1e-3) / 1e9
    tf_s = gu_flops / (gate_up_ms * 1e-3) / 1e12
    if workload in HBM_GRADED:
        roof = {"bound": "hbm", "achieved": round(gb_s, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gb_s / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tf_s, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(tf_s / mfma_peak, 4)}
    roof["traffic"] = measured_traffic(workload, "gate_up_swiglu")
    roof["kernel"] = "gate_up_swiglu"
    roof["kernel_ms"] = round(gate_up_ms, 4)
    roof["algorithmic_bytes"] = gu_bytes
    roof["algorithmic_flops"] = gu_flops
    roof["mfma_dtype"] = mfma_dt
    roof["mfma_frac"] = round(tf_s / mfma_peak, 4)
    roof["hbm_frac"] = round(gb_s / HBM_PEAK_GBS, 4)

    # whole-layer view: touched expert weights (+ gate, shared expert) and
    # flops over the step time
    wb = weight_bytes(cfg)
    A = cfg.T * cfg.k
    layer_w = touched * (3 * cfg.H * cfg.F * wb + 2 * scale_bytes(cfg, cfg.H, cfg.F) + scale_bytes(cfg, cfg.F, cfg.H))
    layer_w += gate_bytes(cfg) + shared_bytes(cfg)
    layer_flops = 6.0 * A * cfg.H * cfg.F + 6.0 * cfg.T * cfg.H * cfg.Fs + 2.0 * cfg.T * cfg.H * cfg.E
    res = {
        "workload": cfg.name, "T": cfg.T, "steps": steps, "warmup": warmup,
        "value": round(cfg.T * steps / elapsed, 1), "ms_per_step": round(ms_per_step, 4),
        "latency_ms": {"p50": round(percentile(lat, 0.5), 4), "p95": round(percentile(lat, 0.95), 4),
                       "max": round(max(lat), 4), "samples": n_lat},
        "roofline": roof,
        "layer": {"touched_experts": touched, "weight_bytes": layer_w,
                  "hbm_frac": round(layer_w / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                  "mfma_frac": round(layer_flops / (ms_per_step * 1e-3) / (mfma_peak * 1e12), 4),
                  "mfma_dtype": mfma_dt, "stages_ms": stages},
        "_data": (d, a8),
    }
    del layer, X, Y
    return res


def ep_bench(args) -> int:
    """The layer with its experts spread over G ranks sharing this GPU
    (dispatch by owner, all-to-all, local experts, return, combine at the
    source): ms per step, per-stage p50/p95, and the all-to-all kernels'
    bandwidth against the HBM peak (their bytes: token rows and records read
    and written on the way out, result rows and the gather index on the way
    back). The single-GPU layer is timed beside it on the same weights."""
    import torch
    import mixture_experts_layer_count_amd as moe
    from synth import get_config, make_layer

    cfg = get_config(args.workload)
    G = args.ep
    d = make_layer(cfg, device="cuda")
    X = d["X"]
    epl = moe.EPLoopback(d, cfg.k, G)
    Y = torch.empty_like(X)
    n_ev = len(moe.EP_STAGES) + 1
    for _ in range(args.warmup):
        epl.forward(X, Y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        epl.forward(X, Y)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    runs = []
    for _ in range(max(10, args.steps)):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        epl.forward(X, Y, events=ev)
        runs.append(ev)
    torch.cuda.synchronize()
    stage = {}
    for i, name in enumerate(moe.EP_STAGES):
        xs = [r[i].elapsed_time(r[i + 1]) for r in runs]
        stage[name] = {"p50": round(percentile(xs, 0.5), 4), "p95": round(percentile(xs, 0.95), 4)}
    step = [r[0].elapsed_time(r[-1]) for r in runs]
    A = cfg.T * cfg.k
    ab = 4 if cfg.act == "f32" else 2
    out_bytes = 2.0 * A * (cfg.H * ab + 16)              # rows + records, read and written
    back_bytes = 2.0 * A * cfg.H * ab + 4.0 * A          # result rows read and written, gather index
    ex_ms, ret_ms = stage["exchange"]["p50"], stage["return"]["p50"]
    layer = moe.MoELayer(d, cfg.k)
    for _ in range(args.warmup):
        layer.forward(X, Y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer.forward(X, Y)
    torch.cuda.synchronize()
    single_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    gbs = out_bytes / (ex_ms * 1e-3) / 1e9
    out = {
        "metric": "MoE-layer tokens/s, experts spread over G ranks on one GPU (loopback all-to-all)",
        "value": round(cfg.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "ranks": G,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "latency_ms": {"p50": round(percentile(step, 0.5), 4), "p95": round(percentile(step, 0.95), 4)},
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "F": cfg.F, "E": cfg.E, "k": cfg.k, "Fs": cfg.Fs,
                   "weights": cfg.w, "experts_per_rank": cfg.E // G},
        "stages_ms": stage,
        "roofline": {"kernel": "ep_exchange (dispatch all-to-all: rows + records)", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": out_bytes,
                     "return_bytes": back_bytes,
                     "return_gb_s": round(back_bytes / (ret_ms * 1e-3) / 1e9, 1) if ret_ms > 0 else None},
        "single_gpu_layer_ms": round(single_ms, 4),
        "data": "synthetic",
    }
    print(json.dumps(out))
    return 0


def dtype_label(cfg, a8: bool) -> str:
    """The type the expert GEMMs multiply in: E4M3 codes on the fp8 matrix
    cores for W8A8; bf16 for bf16 weights and for fp8 or MXFP4 weights that
    are decoded to bf16 beside bf16 activations; fp32 for the fp32 layer.
    The weight and activation formats themselves are in `config`."""
    if cfg.w == "f32":
        return "f32"
    return "fp8" if cfg.w == "fp8" and a8 else "bf16"


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_prefill")
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "tiled", "tiled_a8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-all-configs", action="store_true",
                    help="time only --workload (by default every configuration is timed after it)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--record-traffic", action="store_true",
                    help="write the gate/up HBM traffic record from rocprofv3 counter runs (no GPU)")
    ap.add_argument("--pmc-fetch")
    ap.add_argument("--pmc-write")
    ap.add_argument("--calib-fetch")
    ap.add_argument("--calib-write")
    ap.add_argument("--pmc-kernel", choices=["gate_up", "down"], default="gate_up",
                    help="which GEMM's record --record-traffic writes (bench.py reads the gate/up one)")
    ap.add_argument("--commands", nargs="*", default=[])
    ap.add_argument("--sweep", metavar="WORKLOAD",
                    help="token-count sweep of this workload's layer shape (T = 1 .. --sweep-max-t), every path")
    ap.add_argument("--sweep-max-t", type=int, default=8192)
    ap.add_argument("--ep", type=int, default=0, metavar="G",
                    help="time the layer with its experts spread over G ranks on this GPU (loopback all-to-all)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 kernel-trace run (no GPU)")
    ap.add_argument("--summarize-counter", metavar="DIR",
                    help="print a markdown table of --counter per GEMM kernel from a rocprofv3 --pmc run (no GPU)")
    ap.add_argument("--counter", default="MfmaUtil")
    args = ap.parse_args()
    if args.record_traffic:
        return record_traffic(args)
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_counter:
        return summarize_counter(args)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the MoE layer here runs on a "
              f"single MI355X with all experts resident, and no multi-GPU path is built.", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.sweep:
        return t_sweep(args)
    if args.ep:
        return ep_bench(args)

    from synth import get_config

    cfg = get_config(args.workload)
    m = measure(cfg, args.path, args.steps, args.warmup, args.workload)
    d, a8 = m.pop("_data")
    out = {
        "metric": METRIC,
        "value": m["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_label(cfg, a8),
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "F": cfg.F, "E": cfg.E, "k": cfg.k,
                   "Fs": cfg.Fs, "weights": cfg.w, "shared_weights": cfg.shared_w if cfg.Fs else None,
                   "gate": cfg.wg or cfg.act, "activations": cfg.act, "path": args.path},
        "roofline": m["roofline"],
        "latency_ms": m["latency_ms"],
        "layer": m["layer"],
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, d, cfg.k)
    del d
    torch.cuda.empty_cache()
    if not args.no_all_configs:
        # the other configurations, timed in the same run (each its own
        # seeded layer, freed before the next is drawn)
        table = {}
        for name in ALL_CONFIGS:
            if name == args.workload:
                continue
            c = get_config(name)
            decode = name in DECODE_WORKLOADS
            r = measure(c, "auto", 50 if decode else 20, 10, name)
            r.pop("_data")
            torch.cuda.empty_cache()
            table[name] = {"T": r["T"], "steps": r["steps"], "ms_per_step": r["ms_per_step"],
                           "tokens_per_s": r["value"], "latency_ms": r["latency_ms"],
                           "dominant_kernel": {k2: r["roofline"][k2] for k2 in
                                               ("kernel", "bound", "achieved", "unit", "frac", "kernel_ms",
                                                "mfma_dtype", "mfma_frac", "hbm_frac", "traffic")},
                           "layer_hbm_frac": r["layer"]["hbm_frac"], "layer_mfma_frac": r["layer"]["mfma_frac"],
                           "stages_p50_ms": {s: v["p50"] for s, v in r["layer"]["stages_ms"].items()}}
            print(f"[bench] {name}: {r['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
        out["configs"] = table
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
