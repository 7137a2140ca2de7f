#!/usr/bin/env python3
"""Benchmark of the QoQ W4A8 GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the per-call path over one batch of tokens: per-token
INT8 quantization of the activations, then the W4A8 GEMM against every weight
encoding the workload names (g128 and per-channel for the default Llama-3-8B
fused-QKV decode layer, M=64 K=4096 N=6144). The weights are quantized and
packed once beforehand (the offline stage; it is timed separately and reported
under "offline"). Inputs are resident in HBM when the timed region starts.

Every weight matrix here fits in the 256 MB Infinity Cache, so each step uses
its own copy of every buffer, rotating through enough copies (>= 1 GiB) that a
copy has been evicted before it is used again: the figures are HBM figures.
The steps are replayed from HIP graphs, so the host's launch latency does not
pace the GPU.

Prints one JSON line. "value" is the whole step's algorithmic bytes divided by
its time (GB/s); "roofline" reports the dominant kernel's algorithmic bytes
per launch over its average launch duration, timed with HIP events on the
stream the kernels run on; "cpu_baseline" times the oracle on the host cores
over a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0  # MI355X dense INT8 MFMA (5.0 POPS)

# The default run: the decode layer of the one-line result, and the prefill
# layer of the metric's large-M half (reported in the same line as "large_m").
DEFAULT_WORKLOAD = "llama3_8b_qkv_decode"
LARGE_M_WORKLOAD, LARGE_M_LAYER = "llama3_8b_prefill", "llama3_8b_gate_up_m4096"


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--rotate-mib", type=int, default=1536,
                   help="total size of the rotating buffer copies")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target host time of the oracle's CPU-baseline sample (0: skip)")
    p.add_argument("--kernel-launches", type=int, default=400,
                   help="launches per kernel in the per-kernel timing pass")
    p.add_argument("--layer", default=None,
                   help="layer of a multi-layer workload to time (default: the workload's only layer)")
    p.add_argument("--profile-launches", type=int, default=0,
                   help="instead of timing: launch each kernel of one step this many times on "
                        "cold caches, then a 256 MiB copy as many times (for counter runs)")
    p.add_argument("--all-layers", action="store_true",
                   help="instead of the one-line result: time the GEMMs of every layer of "
                        "every workload and print one line per layer")
    p.add_argument("--formats", action="store_true",
                   help="instead of the one-line result: per layer (of --workload, or of every "
                        "workload with --all-layers), time the per-call path in each weight/"
                        "activation format -- W4A8 g128 and per-channel, W8A8, W4A16 -- and "
                        "print one line per layer (for M > 64 also the vendor library's plain "
                        "INT8 GEMM on the same shape)")
    p.add_argument("--producer", action="store_true",
                   help="instead of the one-line result: time the fused SiLU(gate)*up + "
                        "per-token quantization against the unfused path (torch SiLU*up "
                        "writing h, then qoq_quantize_act) for every down-projection layer")
    p.add_argument("--kv4", action="store_true",
                   help="instead of the one-line result: time KV4 decode attention (4-bit "
                        "cache, SmoothAttention) at the serving shapes next to torch's FP16 "
                        "attention on an FP16 cache of the same shape")
    p.add_argument("--read-probe", action="store_true",
                   help="instead of the one-line result: time plain device-to-device copies "
                        "that move the decode layer's algorithmic bytes (and larger sizes) "
                        "from cold HBM, replayed from a graph like the GEMMs: what one launch "
                        "of that size reaches on this chip")
    p.add_argument("--k-sweep", action="store_true",
                   help="time the layer's GEMMs at K = 128 .. the layer's K (same M and N, same "
                        "seeds) and fit time = fixed + per-K cost; no CPU baseline")
    p.add_argument("--no-large-m", action="store_true",
                   help="leave the large-M half (Llama-3-8B prefill gate_up, M=4096) out of the "
                        "default run's line")
    p.add_argument("--counter-summary", nargs="+", default=None, metavar="DIR",
                   help="instead of timing: read the counter CSVs of rocprofv3 --pmc runs of "
                        "--profile-launches (one directory per pass) and write a per-kernel "
                        "median table for this workload and layer under profiles/")
    p.add_argument("--pmc-summary", nargs="+", default=None, metavar="DIR",
                   help="instead of timing: read rocprofv3 counter CSVs (FETCH_SIZE run, "
                        "WRITE_SIZE run) of a --profile-launches run and write the traffic "
                        "summary for this workload under profiles/")
    return p.parse_args(argv)


def gemm_bytes(mode: int, M: int, N: int, K: int) -> int:
    """Algorithmic HBM bytes of one GEMM launch: packed codes, group or
    per-channel parameters, scales, INT8 activations, row sums, FP16 output."""
    codes = N * K // 2
    if mode == 0:
        params = N * (K // 128)  # one byte per (channel, group): s_g - 1 and z
        extra = 0
    else:
        params = N  # one zero byte per channel
        extra = 4 * M  # row sums
    return codes + params + 2 * N + M * K + 2 * M + extra + 2 * M * N


def act_bytes(M: int, K: int) -> int:
    """Per-token quantization: read FP16 X, write INT8 X, FP16 scale, row sum."""
    return 2 * M * K + M * K + 2 * M + 4 * M


ROOT = os.path.dirname(os.path.abspath(__file__))
# Sources whose kernels the traffic figures describe; a stored figure is used
# only while these files are unchanged.
KERNEL_SOURCES = ("quantized_gemm_qoq_amd/csrc/gemm.hip", "quantized_gemm_qoq_amd/csrc/qoq_device.hpp",
                  "quantized_gemm_qoq_amd/csrc/quantize.hip")
CALIBRATION_MIB = 256


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload: str, layer: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}_{layer}.json")


def stored_traffic(workload: str, layer: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None if there is none or the kernels changed since it was taken."""
    path = traffic_path(workload, layer)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k["hbm_bytes"]


def counter_summary(args, wl, layer) -> int:
    """Median of each hardware counter per kernel over the dispatches of a
    --profile-launches run (one rocprofv3 --pmc pass per directory), written as
    a markdown table to profiles/counters_<workload>_<layer>.md with the
    commands that produced it."""
    import csv
    import glob
    import re
    import statistics

    vals, passes = {}, []
    for d in args.counter_summary:
        names = set()
        for f in glob.glob(os.path.join(d, "**", "*_counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    m = re.search(r"(k_[a-z0-9_]+(<[^>]*>)?)", r["Kernel_Name"])
                    if not m or not m.group(1).startswith(("k_gemm", "k_quantize_act", "k_splitk")):
                        continue
                    names.add(r["Counter_Name"])
                    vals.setdefault((m.group(1), r["Counter_Name"]), []).append(float(r["Counter_Value"]))
        passes.append(sorted(names))
    kernels = sorted({k for k, _ in vals})
    counters = list(dict.fromkeys(c for ps in passes for c in ps))
    lines = [f"# Hardware counters: {wl.name} / {layer.name} (M={layer.M} K={layer.K} N={layer.N})", "",
             "Median per dispatch over the cold-cache launches of `bench.py --profile-launches` "
             "(caches flushed before each launch). SQ_* counters are summed over the shader engines "
             "(SQ_WAVE_CYCLES and SQ_WAIT_* in units of 4 cycles); TCC_* are 128-byte L2 requests "
             "summed over the L2 channels; TA_BUSY_avr averages the compute units' address units; "
             "GRBM_GUI_ACTIVE counts GPU cycles of the dispatch.", "",
             "Commands (one pass per counter set):", ""]
    for ps in passes:
        lines.append(f"    rocprofv3 --kernel-trace --pmc {' '.join(ps)} --output-format csv -d <dir> -- "
                     f"python3 bench.py --workload {wl.name} --layer {layer.name} --profile-launches 3")
    lines += [f"    python3 bench.py --workload {wl.name} --layer {layer.name} --counter-summary <dir> ...",
              "", "| counter | " + " | ".join(f"`{k}`" for k in kernels) + " |",
              "|---|" + "---|" * len(kernels)]
    for c in counters:
        row = [f"{statistics.median(vals[(k, c)]):.0f}" if (k, c) in vals else "" for k in kernels]
        lines.append(f"| {c} | " + " | ".join(row) + " |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    out = os.path.join(ROOT, "profiles", f"counters_{wl.name}_{layer.name}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)
    return 0


def pmc_summary(args, wl, layer) -> int:
    """Turn the counter CSVs of a --profile-launches run into the per-launch HBM
    traffic of each kernel, calibrated by the copy: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch) are each scaled so that the copy of CALIBRATION_MIB reads
    and writes exactly that many bytes."""
    import csv
    import glob
    import statistics

    vals = {}
    for d in args.pmc_summary:
        for f in glob.glob(os.path.join(d, "**", "*_counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    name = r["Kernel_Name"]
                    if "k_gemm" in name or "k_splitk_reduce" in name:
                        # first template argument: the weight format (0 g128, 1 per-channel, 2 INT8)
                        fmt = name.split("<", 1)[1].split(",")[0].split(">")[0].strip()
                        mode = {"0": "g128", "1": "per_channel", "2": "w8a8"}.get(fmt)
                        if mode is None:
                            continue
                        key = ("w4a8_gemm_" + mode) if mode != "w8a8" else "w8a8_gemm"
                        if "k_splitk_reduce" in name:
                            key += "+reduce"  # the split-K plan's second launch, added below
                    elif "k_quantize_act" in name:
                        key = "quantize_act"
                    elif "copyBuffer" in name:
                        key = "copy"
                    else:
                        continue
                    vals.setdefault((key, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    med = {k: statistics.median(v) for k, v in vals.items()}
    cal = CALIBRATION_MIB * 1024.0
    fs = cal / med[("copy", "FETCH_SIZE")]
    ws = cal / med[("copy", "WRITE_SIZE")]
    out = {"workload": wl.name, "layer": layer.name, "M": layer.M, "K": layer.K, "N": layer.N,
           "source_hash": kernel_source_hash(), "source_files": list(KERNEL_SOURCES),
           "calibration": {"copy_MiB": CALIBRATION_MIB,
                           "FETCH_SIZE_KiB": med[("copy", "FETCH_SIZE")],
                           "WRITE_SIZE_KiB": med[("copy", "WRITE_SIZE")],
                           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)},
           "commands": [
               f"rocprofv3 --kernel-trace --pmc FETCH_SIZE --output-format csv -d <dir1> -- "
               f"python3 bench.py --workload {wl.name} --layer {layer.name} --profile-launches 3",
               f"rocprofv3 --kernel-trace --pmc WRITE_SIZE --output-format csv -d <dir2> -- "
               f"python3 bench.py --workload {wl.name} --layer {layer.name} --profile-launches 3",
               f"python3 bench.py --workload {wl.name} --layer {layer.name} --pmc-summary <dir1> <dir2>"],
           "kernels": {}}
    for key in sorted({k for k, _ in med if k != "copy" and not k.endswith("+reduce")}):
        fk, wk = med.get((key, "FETCH_SIZE")), med.get((key, "WRITE_SIZE"))
        if fk is None or wk is None:
            continue
        # a GEMM call of a split-K plan is two launches: both count
        rf, rw = med.get((key + "+reduce", "FETCH_SIZE"), 0.0), med.get((key + "+reduce", "WRITE_SIZE"), 0.0)
        fb, wb = (fk + rf) * 1024 * fs, (wk + rw) * 1024 * ws
        out["kernels"][key] = {"FETCH_SIZE_KiB": fk, "WRITE_SIZE_KiB": wk,
                               "hbm_read_bytes": round(fb), "hbm_write_bytes": round(wb),
                               "hbm_bytes": round(fb + wb)}
        if rf or rw:
            out["kernels"][key]["reduce_FETCH_SIZE_KiB"] = rf
            out["kernels"][key]["reduce_WRITE_SIZE_KiB"] = rw
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(traffic_path(wl.name, layer.name), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out["kernels"]))
    return 0


def run_layer(args, wl, layer):
    """Quantize and pack the layer's weights, then time the step over rotating
    buffer copies; returns the result record (or an int exit code)."""
    from quantized_gemm_qoq_amd import workloads

    import torch

    import quantized_gemm_qoq_amd as qoq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 3
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M, N, K = layer.M, layer.N, layer.K
    modes = [qoq.MODES[m] for m in wl.modes]

    x16, w16 = workloads.generate(layer)
    x_dev, w_dev = x16.to(dev), w16.to(dev)

    # ---- offline stage: quantize + pack once per mode (timed, not in the step)
    offline = {}
    packed = {}
    for mode in modes:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        q, s_c, s_g, z = qoq.qoq_quantize_weights(mode, w_dev)
        blob = qoq.qoq_pack_weights(mode, q, s_g, z)
        torch.cuda.synchronize()
        offline[wl.modes[modes.index(mode)]] = round((time.perf_counter() - t0) * 1e3, 3)
        packed[mode] = (blob, s_c)
        del q, s_g, z

    if args.profile_launches > 0:
        return profile_launches(args, qoq, torch, dev, x_dev, packed, modes, M, N, K)

    # ---- rotating buffer sets
    per_set = 2 * M * K + M * K + 8 * M
    for mode in modes:
        per_set += packed[mode][0].numel() + 2 * N + 2 * M * N
    R = max(2, math.ceil(args.rotate_mib * 2**20 / per_set))
    sets = []
    for r in range(R):
        s = {"x": x_dev.clone(),
             "xq": torch.empty((qoq.qoq_act_bytes(M, K),), dtype=torch.int8, device=dev),
             "s_x": torch.empty((M,), dtype=torch.float16, device=dev),
             "rowsum": torch.empty((M,), dtype=torch.int32, device=dev)}
        for mode in modes:
            blob, s_c = packed[mode]
            s[("blob", mode)] = blob.clone()
            s[("s_c", mode)] = s_c.clone()
            s[("y", mode)] = torch.empty((M, N), dtype=torch.float16, device=dev)
        sets.append(s)

    def step(s):
        qoq.qoq_quantize_act(s["x"], s["xq"], s["s_x"], s["rowsum"])
        for mode in modes:
            rs = s["rowsum"] if mode == qoq.MODE_PER_CHANNEL else None
            qoq.qoq_w4a8_gemm(mode, s["xq"], s["s_x"], rs, s[("blob", mode)], s[("s_c", mode)], N,
                              y=s[("y", mode)])

    # eager warm-up (also loads the code objects)
    for i in range(max(1, args.warmup)):
        step(sets[i % R])
    torch.cuda.synchronize()

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    full = capture(lambda: [step(s) for s in sets])
    rem_n = args.steps % R
    rem = capture(lambda: [step(s) for s in sets[:rem_n]]) if rem_n else None
    reps = args.steps // R

    # graph warm-up
    full.replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        full.replay()
    if rem is not None:
        rem.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    step_bytes = act_bytes(M, K) + sum(gemm_bytes(m, M, N, K) for m in modes)
    step_ops = sum(2 * M * N * K for _ in modes)
    # Decode M is bound by HBM (bytes), large M by the matrix cores (ops); the
    # ridge of 5.0 POPS over 8 TB/s sits near M = 160 for these shapes.
    bound = "hbm" if M <= 162 else "mfma"
    if bound == "hbm":
        metric = ("W4A8 GEMM HBM GB/s (decode M) on the per-call path: per-token INT8 "
                  "quantization + W4A8 GEMM")
        unit = "GB/s"
        value = step_bytes / (ms_per_step * 1e-3) / 1e9
    else:
        metric = ("W4A8 GEMM TOPS (large M) on the per-call path: per-token INT8 "
                  "quantization + W4A8 GEMM")
        unit = "TOPS"
        value = step_ops / (ms_per_step * 1e-3) / 1e12

    # ---- per-kernel timing: HIP events on the stream the kernels run on,
    # bracketing graph replays of back-to-back launches of one kernel over the
    # rotating copies.
    L = max(R, args.kernel_launches // R * R)

    def kernel_avg_us(fn_one):
        g = capture(lambda: [fn_one(sets[i % R]) for i in range(L)])
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / L

    kernels = {}
    act_us = kernel_avg_us(lambda s: qoq.qoq_quantize_act(s["x"], s["xq"], s["s_x"], s["rowsum"]))
    kernels["quantize_act"] = {"avg_us": round(act_us, 3), "bytes": act_bytes(M, K),
                               "GB/s": round(act_bytes(M, K) / act_us / 1e3, 1)}
    for mode in modes:
        name = "w4a8_gemm_" + ("g128" if mode == qoq.MODE_G128 else "per_channel")
        rsk = "rowsum" if mode == qoq.MODE_PER_CHANNEL else None

        def one(s, mode=mode, rsk=rsk):
            qoq.qoq_w4a8_gemm(mode, s["xq"], s["s_x"], s[rsk] if rsk else None,
                              s[("blob", mode)], s[("s_c", mode)], N, y=s[("y", mode)])

        us = kernel_avg_us(one)
        b = gemm_bytes(mode, M, N, K)
        kernels[name] = {"avg_us": round(us, 3), "bytes": b, "GB/s": round(b / us / 1e3, 1),
                         "TOPS": round(2 * M * N * K / us / 1e6, 2)}

    dominant = max((k for k in kernels if k.startswith("w4a8_gemm")),
                   key=lambda k: kernels[k]["avg_us"])
    dk = kernels[dominant]
    traffic = stored_traffic(wl.name, layer.name, dominant)
    if bound == "hbm":
        roofline = {"bound": "hbm", "achieved": dk["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(dk["GB/s"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": dominant, "algorithmic_bytes": dk["bytes"]}
    else:
        roofline = {"bound": "mfma", "achieved": dk["TOPS"], "peak": INT8_PEAK_TOPS,
                    "unit": "TOPS", "frac": round(dk["TOPS"] / INT8_PEAK_TOPS, 4),
                    "traffic": traffic, "kernel": dominant, "algorithmic_ops": 2 * M * N * K,
                    "algorithmic_bytes": dk["bytes"]}

    # ---- CPU baseline: the oracle on the host cores, same step, bounded sample
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(layer, modes, sets[0], bound, args.cpu_seconds)

    out = {
        "metric": metric,
        "value": round(value, 2 if bound == "mfma" else 1),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x uint4 -> int32 (fp16 in/out)",
        "data": describe_data(layer),
        "config": {"workload": wl.name, "layer": layer.name, "description": wl.description,
                   "M": M, "K": K, "N": N,
                   "modes": list(wl.modes), "parallelism": "single GPU",
                   "rotating_copies": R, "graph_replay": True},
        "step_bytes": step_bytes,
        "step_TOPS": round(step_ops / (ms_per_step * 1e-3) / 1e12, 2),
        "kernels": kernels,
        "roofline": roofline,
        "offline_ms": offline,
        "cpu_baseline": cpu,
    }
    return out


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: the path runs on one GPU only (asked for --gpus {args.gpus}); "
              "no multi-GPU figure is produced.", file=sys.stderr)
        return 2
    if args.steps < 1:
        print("bench.py: --steps must be >= 1", file=sys.stderr)
        return 2

    from quantized_gemm_qoq_amd import workloads

    wl = workloads.WORKLOADS[args.workload]
    if args.layer is None and len(wl.layers) != 1:
        layer_list = ", ".join(l.name for l in wl.layers)
        print(f"bench.py: workload {wl.name} has several layers ({layer_list}); "
              "name one with --layer", file=sys.stderr)
        return 2
    layers = [l for l in wl.layers if args.layer in (None, l.name)]
    if not layers:
        print(f"bench.py: no layer {args.layer} in workload {wl.name}", file=sys.stderr)
        return 2
    layer = layers[0]
    if args.pmc_summary:
        return pmc_summary(args, wl, layer)
    if args.counter_summary:
        return counter_summary(args, wl, layer)

    if args.kv4:
        for name, B, Hq, H, T in KV4_SHAPES:
            out = kv4_compare(args, name, B, Hq, H, T)
            if isinstance(out, int):
                return out
            print(json.dumps(out), flush=True)
        return 0
    if args.producer:
        for wl2 in workloads.WORKLOADS.values():
            for layer2 in wl2.layers:
                if "down" in layer2.name:
                    out = producer_compare(args, layer2)
                    if isinstance(out, int):
                        return out
                    print(json.dumps(out), flush=True)
        for M2, I2 in SILU_SPLIT_SHAPES:
            layer2 = workloads.Layer(f"silu_m{M2}_i{I2}", M=M2, K=I2, N=16, seed=3100 + M2)
            out = producer_compare(args, layer2)
            if isinstance(out, int):
                return out
            print(json.dumps(out), flush=True)
        seen = set()
        for wl2 in workloads.WORKLOADS.values():
            for layer2 in wl2.layers:
                if ("qkv" in layer2.name or "gate_up" in layer2.name) and (layer2.M, layer2.K) not in seen:
                    seen.add((layer2.M, layer2.K))
                    out = rmsnorm_compare(args, layer2)
                    if isinstance(out, int):
                        return out
                    print(json.dumps(out), flush=True)
        return 0
    if args.read_probe:
        return read_probe(args, wl, layer)
    if args.k_sweep:
        return k_sweep(args, wl, layer)
    if args.formats:
        todo = [(w, l) for w in (workloads.WORKLOADS.values() if args.all_layers else [wl])
                for l in w.layers if args.all_layers or args.layer in (None, l.name)]
        for wl2, layer2 in todo:
            out = format_compare(args, wl2, layer2)
            if isinstance(out, int):
                return out
            print(json.dumps(out), flush=True)
        return 0
    if args.all_layers:
        for wl2 in workloads.WORKLOADS.values():
            for layer2 in wl2.layers:
                out = run_layer(args, wl2, layer2)
                if isinstance(out, int):
                    return out
                k = {n: {f: v[f] for f in ("avg_us", "GB/s", "TOPS") if f in v}
                     for n, v in out["kernels"].items()}
                print(json.dumps({"workload": wl2.name, "layer": layer2.name, "M": layer2.M,
                                  "K": layer2.K, "N": layer2.N, "kernels": k}), flush=True)
        return 0
    out = run_layer(args, wl, layer)
    if isinstance(out, int):
        return out
    if args.workload == DEFAULT_WORKLOAD and args.layer is None and not args.no_large_m:
        # The metric's large-M half: TOPS and % of INT8 peak on a prefill layer.
        wl2 = workloads.WORKLOADS[LARGE_M_WORKLOAD]
        layer2 = [l for l in wl2.layers if l.name == LARGE_M_LAYER][0]
        big = run_layer(args, wl2, layer2)
        if isinstance(big, int):
            return big
        out["large_m"] = {k: big[k] for k in ("metric", "value", "unit", "ms_per_step", "dtype",
                                              "data", "config", "step_TOPS", "kernels", "roofline",
                                              "cpu_baseline")}
    print(json.dumps(out))
    return 0


# Decode attention at the pages' serving point (1024 input + 512 output tokens:
# 1536 cached tokens at the last step), head dimension 128.
# Few-row inputs of a down projection (Llama-2-7B's 11008, Llama-3-8B's 14336,
# Qwen1.5-72B's 24576 inputs) around the split-row policy's edges.
SILU_SPLIT_SHAPES = ((1, 24576), (16, 14336), (32, 14336), (16, 11008), (64, 14336))

KV4_SHAPES = (("llama3_8b_b64", 64, 32, 8, 1536), ("llama3_8b_b16", 16, 32, 8, 1536),
              ("qwen15_72b_b16", 16, 64, 64, 1536), ("hq64_h8_b16", 16, 64, 8, 1536),
              ("llama3_8b_b16_t8192", 16, 32, 8, 8192))


def kv4_compare(args, name, B, Hq, H, T):
    """KV4 decode attention vs torch FP16 attention, cold caches (rotating copies)."""
    import torch

    import quantized_gemm_qoq_amd as qoq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 3
    dev = torch.device("cuda:0")
    d = qoq.HEAD_DIM
    g = torch.Generator(device="cpu")
    g.manual_seed(8000 + B + Hq)
    k = torch.randn(B, T, H, d, generator=g).to(torch.float16).to(dev)
    v = torch.randn(B, T, H, d, generator=g).to(torch.float16).to(dev)
    q = torch.randn(B, Hq, d, generator=g).to(torch.float16).to(dev)
    lam = qoq.qoq_kv4_smooth_scales(k[0])
    lens = torch.full((B,), T, dtype=torch.int32, device=dev)
    kv4_bytes = B * H * T * (2 * d // 2 + 2 * 3)  # codes, scales, zeros of K and V
    R = max(2, math.ceil(args.rotate_mib * 2**20 / kv4_bytes))
    caches = []
    for _ in range(R):
        c = qoq.KV4Cache(B, H, T, dev, lam)
        c.append(k, v, 0)
        caches.append(c)
    ws = torch.empty((max(16, qoq.load_library().qoq_kv4_attention_workspace_bytes(B, Hq, H, d, T)),),
                     dtype=torch.uint8, device=dev)
    outs = [torch.empty((B, Hq, d), dtype=torch.float16, device=dev) for _ in range(R)]
    fp16_bytes = 2 * B * H * T * d * 2
    R16 = max(2, math.ceil(args.rotate_mib * 2**20 / fp16_bytes))
    kvs = [(k.permute(0, 2, 1, 3).contiguous(), v.permute(0, 2, 1, 3).contiguous()) for _ in range(R16)]
    q4 = q.view(B, Hq, 1, d)
    del k, v

    def avg_us(fns, launches):
        for f in fns[:2]:
            f()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(launches):
                fns[i % len(fns)]()
        gr.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / launches

    L = max(R, args.kernel_launches // R * R)
    us4 = avg_us([lambda i=i: caches[i].attention(q, lens, o=outs[i], workspace=ws) for i in range(R)], L)
    sdpa = torch.nn.functional.scaled_dot_product_attention
    try:
        L16 = max(R16, args.kernel_launches // R16 * R16)
        us16 = avg_us([lambda i=i: sdpa(q4, kvs[i][0], kvs[i][1], enable_gqa=True) for i in range(R16)], L16)
    except Exception as e:  # an FP16 attention path torch lacks here: report without it
        print(f"bench.py: torch FP16 attention not timed ({e})", file=sys.stderr)
        us16 = None
    alg = kv4_bytes + 2 * 2 * B * Hq * d + 4 * B + 2 * H * d
    return {"shape": name, "B": B, "Hq": Hq, "H": H, "T": T, "kv4_us": round(us4, 3),
            "kv4_GBs": round(alg / us4 / 1e3, 1), "kv4_frac_of_hbm": round(alg / us4 / 1e3 / HBM_PEAK_GBS, 3),
            "kv4_bytes": alg, "fp16_torch_us": None if us16 is None else round(us16, 3),
            "fp16_cache_bytes": fp16_bytes,
            "speedup_vs_fp16": None if us16 is None else round(us16 / us4, 2)}


def producer_compare(args, layer):
    """Fused producer vs unfused path for the input of a down projection with
    M rows and I = K inputs; the gate_up matrix [M, 2I] is synthetic N(0,1)
    FP16 (seeded with the layer's seed). HBM figures over rotating copies."""
    import torch

    import quantized_gemm_qoq_amd as qoq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 3
    dev = torch.device("cuda:0")
    M, I = layer.M, layer.K
    g = torch.Generator(device="cpu")
    g.manual_seed(layer.seed)
    gu = torch.randn(M, 2 * I, generator=g).to(torch.float16).to(dev)
    per = 2 * M * 2 * I + 2 * M * I + M * I
    R = max(2, math.ceil(args.rotate_mib * 2**20 / per))
    sets = [{"gu": gu.clone(), "h": torch.empty((M, I), dtype=torch.float16, device=dev),
             "xq": torch.empty((qoq.qoq_act_bytes(M, I),), dtype=torch.int8, device=dev),
             "s_x": torch.empty((M,), dtype=torch.float16, device=dev),
             "rs": torch.empty((M,), dtype=torch.int32, device=dev)} for _ in range(R)]
    L = max(R, args.kernel_launches // R * R)

    def fused(st):
        qoq.qoq_silu_mul_quantize_act(st["gu"], st["xq"], st["s_x"], st["rs"])

    def one_pass(st):
        qoq.qoq_silu_mul_quantize_act(st["gu"], st["xq"], st["s_x"], st["rs"], workspace=None)

    def unfused(st):
        torch.mul(torch.nn.functional.silu(st["gu"][:, :I]), st["gu"][:, I:], out=st["h"])
        qoq.qoq_quantize_act(st["h"], st["xq"], st["s_x"], st["rs"])

    def avg_us(fn):
        for st in sets[:2]:
            fn(st)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(L):
                fn(sets[i % R])
        gr.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / L

    f_us, u_us = avg_us(fused), avg_us(unfused)
    f_bytes = 4 * M * I + M * I + 6 * M  # read gate_up, write codes, scale, row sum
    out = {"layer": layer.name, "M": M, "I": I, "fused_us": round(f_us, 3),
           "unfused_us": round(u_us, 3), "speedup": round(u_us / f_us, 2),
           "fused_GBs": round(f_bytes / f_us / 1e3, 1),
           "fused_frac_of_hbm": round(f_bytes / f_us / 1e3 / HBM_PEAK_GBS, 3)}
    if qoq.load_library().qoq_silu_mul_workspace_bytes(M, I) > 0:
        out["split_rows"] = True  # fused_us is the split-row path; the one-pass kernel beside it
        out["one_pass_us"] = round(avg_us(one_pass), 3)
    return out


def rmsnorm_compare(args, layer, eps=1e-5):
    """Fused RMSNorm + per-token quantization vs torch's FP16 rms_norm writing
    y and then qoq_quantize_act, for the input [M, K] of a qkv or gate_up
    layer (x synthetic N(0,1) FP16, gamma U(0.5, 1.5)). HBM figures over
    rotating copies."""
    import torch

    import quantized_gemm_qoq_amd as qoq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 3
    dev = torch.device("cuda:0")
    M, K = layer.M, layer.K
    g = torch.Generator(device="cpu")
    g.manual_seed(layer.seed + 77)
    x = torch.randn(M, K, generator=g).to(torch.float16).to(dev)
    gamma = (torch.rand(K, generator=g) + 0.5).to(torch.float16).to(dev)
    per = 2 * M * K * 2 + M * K
    R = max(2, math.ceil(args.rotate_mib * 2**20 / per))
    sets = [{"x": x.clone(), "y": torch.empty((M, K), dtype=torch.float16, device=dev),
             "xq": torch.empty((qoq.qoq_act_bytes(M, K),), dtype=torch.int8, device=dev),
             "s_x": torch.empty((M,), dtype=torch.float16, device=dev),
             "rs": torch.empty((M,), dtype=torch.int32, device=dev)} for _ in range(R)]
    L = max(R, args.kernel_launches // R * R)

    def fused(st):
        qoq.qoq_rmsnorm_quantize_act(st["x"], gamma, eps, st["xq"], st["s_x"], st["rs"])

    def unfused(st):
        st["y"].copy_(torch.nn.functional.rms_norm(st["x"], (K,), gamma, eps))
        qoq.qoq_quantize_act(st["y"], st["xq"], st["s_x"], st["rs"])

    def avg_us(fn):
        for st in sets[:2]:
            fn(st)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(L):
                fn(sets[i % R])
        gr.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / L

    f_us, u_us = avg_us(fused), avg_us(unfused)
    f_bytes = 2 * M * K + 2 * K + M * K + 6 * M  # read x and gamma, write codes, scale, row sum
    return {"producer": "rmsnorm", "layer_input_of": layer.name, "M": M, "K": K,
            "fused_us": round(f_us, 3), "unfused_us": round(u_us, 3), "speedup": round(u_us / f_us, 2),
            "fused_GBs": round(f_bytes / f_us / 1e3, 1),
            "fused_frac_of_hbm": round(f_bytes / f_us / 1e3 / HBM_PEAK_GBS, 3)}


FORMATS = ("w4a8_g128", "w4a8_per_channel", "w8a8", "w4a16_g128")


def fit_line(xs, ys):
    """Least-squares line y = a + b x through the points; returns (a, b)."""
    n = len(xs)
    if n < 2 or len(ys) != n:
        raise ValueError("a line needs at least two points")
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    if sxx == 0:
        raise ValueError("a line needs two distinct x values")
    b = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sxx
    return my - b * mx, b


def k_sweep(args, wl, layer):
    """The layer's GEMMs at K = 128, 256, ... up to its own K (same M, N and
    seeds), timed like the default run, one line per K; then, per GEMM, the
    least-squares line time = fixed + slope * K. The intercept is what a
    launch of this M and N costs before its time grows with K; the slope
    gives the rate at which the K-dependent bytes (codes, group parameters
    and activations) stream, and, above the ridge (M > 162), the rate of the
    K-dependent matrix work. Above the ridge the sweep starts at K = 512, the
    smallest K the large-block kernel takes, so that one kernel spans it."""
    import dataclasses

    args.cpu_seconds = 0
    ks, times = [], {}
    K = 512 if layer.M > 162 else 128
    while K <= layer.K:
        sub = dataclasses.replace(layer, name=f"{layer.name}_k{K}", K=K)
        out = run_layer(args, wl, sub)
        if isinstance(out, int):
            return out
        ks.append(K)
        line = {"probe": "k sweep", "layer": layer.name, "M": layer.M, "N": layer.N, "K": K}
        for name, v in out["kernels"].items():
            times.setdefault(name, []).append(v["avg_us"])
            line[name + "_us"] = v["avg_us"]
        print(json.dumps(line), flush=True)
        K *= 2
    for name, ts in times.items():
        fixed, slope = fit_line(ks, ts)
        fit = {"probe": "k sweep fit", "layer": layer.name, "kernel": name,
               "fixed_us": round(fixed, 3), "us_per_1024_k": round(slope * 1024, 3)}
        if name.startswith("w4a8_gemm"):
            mode = 0 if name.endswith("g128") else 1
            per_k = (gemm_bytes(mode, layer.M, layer.N, 2 * 128) -
                     gemm_bytes(mode, layer.M, layer.N, 128)) / 128  # bytes per unit of K
            fit["streamed_GB/s"] = round(per_k / slope / 1e3, 1)
            fit["k_work_TOPS"] = round(2 * layer.M * layer.N / slope / 1e6, 1)
        print(json.dumps(fit), flush=True)
    return 0


def read_probe(args, wl, layer):
    """Copies that move as many bytes as one GEMM launch of the layer (and
    larger ones), over rotating source and destination buffers (cold HBM),
    replayed from a graph and timed with HIP events like the GEMMs. A copy
    of S bytes reads S and writes S; one line per size with the bytes moved
    per launch, the time and the rate."""
    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 3
    dev = torch.device("cuda:0")
    layer_bytes = max(gemm_bytes(m, layer.M, layer.N, layer.K) for m in (0, 1))
    for moved in (layer_bytes, 2 * layer_bytes, 100 * 2**20, 400 * 2**20):
        size = (moved // 2 + 255) // 256 * 256
        R = max(2, math.ceil(args.rotate_mib * 2**20 / (2 * size)))
        src = [torch.empty(size, dtype=torch.uint8, device=dev).fill_(i % 251) for i in range(R)]
        dst = [torch.empty(size, dtype=torch.uint8, device=dev) for _ in range(R)]
        L = max(R, args.kernel_launches // R * R)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(L):
                dst[i % R].copy_(src[i % R])
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / L
        print(json.dumps({"probe": "device copy", "layer": layer.name, "bytes_moved": 2 * size,
                          "copy_bytes": size, "rotating_copies": R, "launches": L,
                          "avg_us": round(us, 3), "GB/s": round(2 * size / us / 1e3, 1),
                          "frac_of_8TBps": round(2 * size / us / 1e3 / 8000, 3)}), flush=True)
        del src, dst, g
        torch.cuda.empty_cache()
    return 0


def format_compare(args, wl, layer):
    """Time one layer's per-call path in every format on the same synthetic
    weights and activations: the kernels alone and the whole call (W4A8 and
    W8A8 quantize the FP16 activations per token first; W4A16 takes them as
    they are). Each format rotates through its own buffer copies (>= the
    --rotate-mib total), so the figures are HBM figures."""
    from quantized_gemm_qoq_amd import workloads

    import torch

    import quantized_gemm_qoq_amd as qoq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 3
    dev = torch.device("cuda:0")
    M, N, K = layer.M, layer.N, layer.K
    x16, w16 = workloads.generate(layer)
    x_dev, w_dev = x16.to(dev), w16.to(dev)
    res = {"workload": wl.name, "layer": layer.name, "M": M, "K": K, "N": N, "formats": {}}

    def avg_us(fns, launches):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(launches):
                fns[i % len(fns)]()
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / launches

    for fmt in FORMATS:
        mode = {"w4a8_g128": qoq.MODE_G128, "w4a8_per_channel": qoq.MODE_PER_CHANNEL,
                "w8a8": qoq.W8A8, "w4a16_g128": qoq.MODE_G128}[fmt]
        pw = qoq.PackedWeight(mode, w_dev)
        quantized = fmt != "w4a16_g128"
        per = pw.blob.numel() + 2 * M * K + 2 * M * N + (M * K if quantized else 0)
        R = max(2, math.ceil(args.rotate_mib * 2**20 / per))
        L = max(R, args.kernel_launches // R * R)
        sets = []
        for _ in range(R):
            st = {"x": x_dev.clone(), "blob": pw.blob.clone(),
                  "y": torch.empty((M, N), dtype=torch.float16, device=dev)}
            if quantized:
                st["xq"], st["s_x"], st["rs"] = qoq.qoq_quantize_act(
                    x_dev, want_rowsum=mode == qoq.MODE_PER_CHANNEL)
            sets.append(st)
        ws = None
        if quantized:
            ws = qoq.gemm_workspace(mode, M, N, K, dev)

        def gemm(st):
            if fmt == "w4a16_g128":
                qoq.qoq_w4a16_gemm(mode, st["x"], st["blob"], pw.s_c, N, y=st["y"])
            elif fmt == "w8a8":
                qoq.qoq_w8a8_gemm(st["xq"], st["s_x"], st["blob"], pw.s_c, N, y=st["y"], workspace=ws)
            else:
                qoq.qoq_w4a8_gemm(mode, st["xq"], st["s_x"], st["rs"], st["blob"], pw.s_c, N,
                                  y=st["y"], workspace=ws)

        def call(st):
            if quantized:
                qoq.qoq_quantize_act(st["x"], st["xq"], st["s_x"], st["rs"])
            gemm(st)

        for st in sets[:2]:
            call(st)
        torch.cuda.synchronize()
        g_us = avg_us([lambda st=st: gemm(st) for st in sets], L)
        c_us = avg_us([lambda st=st: call(st) for st in sets], L)
        res["formats"][fmt] = {"gemm_us": round(g_us, 3), "call_us": round(c_us, 3),
                               "weight_MB": round(pw.blob.numel() / 1e6, 2),
                               "gemm_TOPS": round(2 * M * N * K / g_us / 1e6, 1),
                               "call_TOPS": round(2 * M * N * K / c_us / 1e6, 1)}
        del sets, pw
        torch.cuda.empty_cache()
    best = min(res["formats"], key=lambda f: res["formats"][f]["call_us"])
    res["fastest_call"] = best
    if M > 64:
        # Context for the matrix-core ceiling: the vendor library's plain INT8
        # GEMM (torch._int_mm: INT8 [M,K] x INT8 [K,N] -> INT32, no rescale)
        # on random INT8 operands of the same shape, over rotating copies.
        per = M * K + N * K + 4 * M * N
        R = max(2, math.ceil(args.rotate_mib * 2**20 / per))
        L = max(R, args.kernel_launches // R * R)
        g = torch.Generator(device="cpu")
        g.manual_seed(layer.seed)
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, generator=g).to(dev)
        b = torch.randint(-127, 128, (N, K), dtype=torch.int8, generator=g).to(dev)
        sets = [(a.clone(), b.clone(), torch.empty((M, N), dtype=torch.int32, device=dev))
                for _ in range(R)]
        for st in sets[:2]:
            torch._int_mm(st[0], st[1].t(), out=st[2])
        torch.cuda.synchronize()
        v_us = avg_us([lambda st=st: torch._int_mm(st[0], st[1].t(), out=st[2]) for st in sets], L)
        res["vendor_int8_gemm"] = {"gemm_us": round(v_us, 3),
                                   "gemm_TOPS": round(2 * M * N * K / v_us / 1e6, 1)}
        del sets
        torch.cuda.empty_cache()
        # ... and its FP8 GEMM (torch._scaled_mm, e4m3 operands, unit scales,
        # BF16 out), whose dense peak on this chip equals the INT8 one.
        try:
            per = M * K + N * K + 2 * M * N
            R = max(2, math.ceil(args.rotate_mib * 2**20 / per))
            L = max(R, args.kernel_launches // R * R)
            a8 = (torch.randn((M, K), generator=g) * 0.5).to(dev).to(torch.float8_e4m3fn)
            b8 = (torch.randn((N, K), generator=g) * 0.5).to(dev).to(torch.float8_e4m3fn)
            one = torch.ones((), device=dev)
            sets = [(a8.clone(), b8.clone(), torch.empty((M, N), dtype=torch.bfloat16, device=dev))
                    for _ in range(R)]

            def fp8(st):
                torch._scaled_mm(st[0], st[1].t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16,
                                 out=st[2])

            for st in sets[:2]:
                fp8(st)
            torch.cuda.synchronize()
            f_us = avg_us([lambda st=st: fp8(st) for st in sets], L)
            res["vendor_fp8_gemm"] = {"gemm_us": round(f_us, 3),
                                      "gemm_TFLOPS": round(2 * M * N * K / f_us / 1e6, 1)}
            del sets
        except (RuntimeError, TypeError) as e:  # no FP8 GEMM in this build of the vendor library
            res["vendor_fp8_gemm"] = {"error": str(e)[:200]}
        torch.cuda.empty_cache()
    return res


def describe_data(layer) -> str:
    w = f"W ~ N(0,{layer.w_sigma})"
    if layer.w_outliers:
        w += f" with {layer.w_outliers} input channels x{layer.w_outlier_scale:g}"
    x = "X ~ N(0,1)" if layer.x_kind == "normal" else "X = SiLU(A)*B, A,B ~ N(0,1)"
    if layer.x_outliers:
        x += f" with {layer.x_outliers} channels x{layer.x_outlier_scale:g}"
    return f"synthetic, seeded ({layer.seed}): {w}, {x}; FP16"


def profile_launches(args, qoq, torch, dev, x_dev, packed, modes, M, N, K) -> int:
    """Launch every kernel of one step `--profile-launches` times, each on cold
    caches (a 512 MiB fill in between evicts the L2s and the Infinity Cache),
    then the calibration copy of CALIBRATION_MIB as many times. Nothing is
    timed: this is the program that counter runs profile."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    xq = torch.empty((qoq.qoq_act_bytes(M, K),), dtype=torch.int8, device=dev)
    s_x = torch.empty((M,), dtype=torch.float16, device=dev)
    rowsum = torch.empty((M,), dtype=torch.int32, device=dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    for i in range(args.profile_launches):
        flush.fill_(i & 0xFF)
        qoq.qoq_quantize_act(x_dev, xq, s_x, rowsum)
        for mode in modes:
            blob, s_c = packed[mode]
            flush.fill_(i & 0xFF)
            qoq.qoq_w4a8_gemm(mode, xq, s_x, rowsum if mode == qoq.MODE_PER_CHANNEL else None,
                              blob, s_c, N, y=y)
    src = torch.full((CALIBRATION_MIB << 20,), 1, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for i in range(args.profile_launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile_launches": args.profile_launches, "M": M, "N": N, "K": K,
                      "modes": [int(m) for m in modes], "calibration_MiB": CALIBRATION_MIB}))
    return 0


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(layer, modes, s, bound, seconds):
    """Time the oracle (the plain C reference, as it stands) on the host cores
    over the same step on the first `rows` token rows of the workload, with
    `rows` chosen so that the sample takes about `seconds` (all M rows where
    that fits), and spot-check the GPU's outputs of this buffer set against it.
    The rate is the sample's own algorithmic bytes (or ops) over its time."""
    import numpy as np
    import torch

    import oracle
    from quantized_gemm_qoq_amd import workloads

    x16, w16 = workloads.generate(layer)
    M, N, K = layer.M, layer.N, layer.K
    xb_all = x16.numpy().view(np.uint16)
    wb = w16.numpy().view(np.uint16)
    prepared = {mode: oracle.quantize_weights(mode, wb) for mode in modes}

    def one_step(rows):
        xq, s_x, _ = oracle.quantize_act(np.ascontiguousarray(xb_all[:rows]))
        ys = {}
        for mode in modes:
            wq = prepared[mode]
            acc = oracle.gemm(mode, xq, wq["q"], wq["s_g"], wq["z"])
            ys[mode] = oracle.epilogue(acc, s_x, wq["s_c"])
        return ys

    # Size the sample: one probe step on a few rows gives the cost per row.
    probe = min(M, 4)
    t0 = time.perf_counter()
    one_step(probe)
    per_row = (time.perf_counter() - t0) / probe
    rows = int(max(1, min(M, seconds / 2 / max(per_row, 1e-9))))
    reps = 0
    t0 = time.perf_counter()
    while True:
        ys = one_step(rows)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    ok = True
    for mode in modes:
        yg = s[("y", mode)][:rows].cpu().view(torch.int16).numpy().view(np.float16).astype(np.float64)
        ok &= bool(np.abs(yg - ys[mode]).max() <= 1e-3 * np.abs(ys[mode]).max())
    if bound == "hbm":
        work = act_bytes(rows, K) + sum(gemm_bytes(m, rows, N, K) for m in modes)
        value, unit = work / dt / 1e9, "GB/s"
    else:
        work = sum(2 * rows * N * K for _ in modes)
        value, unit = work / dt / 1e12, "TOPS"
    return {"value": round(value, 4), "unit": unit,
            "cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{reps} step(s) on the first {rows} of {M} token rows (per-token "
                      f"quantization + {len(modes)} GEMM(s) + epilogue over all N={N} "
                      f"channels), {dt * 1e3:.1f} ms each; rate = the sample's algorithmic "
                      f"{'bytes' if bound == 'hbm' else 'ops'} over its time",
            "ms_per_sample_step": round(dt * 1e3, 2),
            "gpu_matches_oracle": ok}


if __name__ == "__main__":
    sys.exit(main())
