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


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="llama3_8b_qkv_decode")
    p.add_argument("--rotate-mib", type=int, default=1536,
                   help="total size of the rotating buffer copies")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target host time of the oracle's CPU-baseline sample (0: skip)")
    p.add_argument("--kernel-launches", type=int, default=400,
                   help="launches per kernel in the per-kernel timing pass")
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


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path is single-GPU and no multi-GPU figure is produced.", file=sys.stderr)
        return 2
    if args.steps < 1:
        print("bench.py: --steps must be >= 1", file=sys.stderr)
        return 2

    import torch

    import quantized_gemm_qoq_amd as qoq
    from quantized_gemm_qoq_amd import workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 3
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.WORKLOADS[args.workload]
    if len(wl.layers) != 1:
        layer_list = ", ".join(l.name for l in wl.layers)
        print(f"bench.py: workload {wl.name} has several layers ({layer_list}); "
              "the benchmark times single-layer workloads", file=sys.stderr)
        return 2
    layer = wl.layers[0]
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
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

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
    bound = "hbm" if M <= 162 else "mfma"
    if bound == "hbm":
        roofline = {"bound": "hbm", "achieved": dk["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(dk["GB/s"] / HBM_PEAK_GBS, 4), "traffic": None,
                    "kernel": dominant}
    else:
        roofline = {"bound": "mfma", "achieved": dk["TOPS"], "peak": INT8_PEAK_TOPS,
                    "unit": "TOPS", "frac": round(dk["TOPS"] / INT8_PEAK_TOPS, 4),
                    "traffic": None, "kernel": dominant}

    # ---- CPU baseline: the oracle on the host cores, same step, bounded sample
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(layer, modes, sets[0], step_bytes, args.cpu_seconds)

    out = {
        "metric": "W4A8 GEMM HBM GB/s (decode M) on the per-call path: per-token INT8 "
                  "quantization + W4A8 GEMM",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x uint4 -> int32 (fp16 in/out)",
        "data": "synthetic (seeded N(0,0.02) weights with 0.5% x10 input channels, N(0,1) activations)",
        "config": {"workload": wl.name, "description": wl.description, "M": M, "K": K, "N": N,
                   "modes": list(wl.modes), "parallelism": "single GPU",
                   "rotating_copies": R, "graph_replay": True},
        "step_bytes": step_bytes,
        "step_TOPS": round(step_ops / (ms_per_step * 1e-3) / 1e12, 2),
        "kernels": kernels,
        "roofline": roofline,
        "offline_ms": offline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))
    return 0


def cpu_baseline(layer, modes, s, step_bytes, seconds):
    """Time the oracle (the plain C reference, as it stands) on the host over
    whole steps of the same workload until `seconds` have passed (at least one
    step), and spot-check the GPU's last outputs of this buffer set against it."""
    import numpy as np
    import torch

    import oracle
    from quantized_gemm_qoq_amd import workloads

    x16, w16 = workloads.generate(layer)
    xb = x16.numpy().view(np.uint16)
    wb = w16.numpy().view(np.uint16)
    prepared = {}
    for mode in modes:
        wq = oracle.quantize_weights(mode, wb)
        prepared[mode] = wq
    reps = 0
    t0 = time.perf_counter()
    while True:
        xq, s_x, rowsum = oracle.quantize_act(xb)
        ys = {}
        for mode in modes:
            wq = prepared[mode]
            acc = oracle.gemm(mode, xq, wq["q"], wq["s_g"], wq["z"])
            ys[mode] = oracle.epilogue(acc, s_x, wq["s_c"])
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    ok = True
    for mode in modes:
        yg = s[("y", mode)].cpu().view(torch.int16).numpy().view(np.float16).astype(np.float64)
        ok &= bool(np.abs(yg - ys[mode]).max() <= 1e-3 * np.abs(ys[mode]).max())
    return {"value": round(step_bytes / dt / 1e9, 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} whole step(s) of the same workload (per-token quantization + "
                      f"{len(modes)} GEMM(s) + epilogue), {dt * 1e3:.1f} ms each",
            "ms_per_step": round(dt * 1e3, 2),
            "gpu_matches_oracle": ok}


if __name__ == "__main__":
    sys.exit(main())
