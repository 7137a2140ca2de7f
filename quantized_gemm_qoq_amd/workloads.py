"""Seeded synthetic inputs shaped like the layers the QServe pages evaluate.

This module only draws random FP16 tensors; it holds none of the method's
arithmetic, so that the tests, the benchmark and the oracle can all consume
the same inputs without sharing any quantization or GEMM code.

The pages evaluate Llama-3-8B and Qwen1.5-72B serving (1024 input / 512 output
tokens, 64 requests). Trained weights and evaluation datasets are not
available, so every tensor is drawn here instead, with those models' layer
shapes:

  * W[N,K] ~ N(0, sigma) in fp32, optionally with `w_outliers` input channels
    (columns of W, chosen by a random permutation from the same generator)
    multiplied by `w_outlier_scale`, then cast to FP16.
  * X[M,K] ~ N(0, 1) in fp32 (or SiLU(A) * B with A, B ~ N(0,1) i.i.d. for the
    MLP down-projection input), optionally with `x_outliers` channels
    multiplied by `x_outlier_scale`, then cast to FP16.

One `torch.Generator` seeded with the layer's seed draws, in this order: W, the
W outlier permutation, X (at `m_gen` rows, of which the first M are used), the
X outlier permutation.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    M: int
    K: int
    N: int
    seed: int
    w_sigma: float = 0.02
    w_outliers: int = 0
    w_outlier_scale: float = 1.0
    x_kind: str = "normal"  # "normal" or "silu_mul"
    x_outliers: int = 0
    x_outlier_scale: float = 1.0
    m_gen: int = 0  # rows drawn for X (0: M); the first M are used

    @property
    def rows_drawn(self) -> int:
        return self.m_gen or self.M


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    modes: Tuple[str, ...]
    layers: Tuple[Layer, ...]


def _qwen_layers(M: int) -> Tuple[Layer, ...]:
    # Qwen1.5-72B: hidden 8192, intermediate 24576, 64 heads (fused qkv 3*8192).
    shapes = [("qkv", 8192, 24576, 5000), ("o_proj", 8192, 8192, 5001),
              ("gate_up", 8192, 49152, 5002), ("down", 24576, 8192, 5003)]
    return tuple(Layer(f"qwen72b_{n}_m{M}", M=M, K=K, N=N, seed=s, w_sigma=0.015, m_gen=1024)
                 for n, K, N, s in shapes)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", "tiny QoQ W4A8 GEMM, M=8 K=512 N=256", ("g128",),
        (Layer("tiny", M=8, K=512, N=256, seed=1000),)),
    "llama3_8b_qkv_decode": Workload(
        "llama3_8b_qkv_decode",
        "Llama-3-8B fused QKV projection at decode, M=64 K=4096 N=6144 (4096+1024+1024)",
        ("g128", "per_channel"),
        # 0.5% of the 4096 input channels (20) carry x10 weights.
        (Layer("llama3_8b_qkv_m64", M=64, K=4096, N=6144, seed=2000,
               w_outliers=20, w_outlier_scale=10.0),)),
    "llama3_8b_mlp_m256": Workload(
        "llama3_8b_mlp_m256", "Llama-3-8B MLP at M=256: gate_up K=4096 N=28672, down K=14336 N=4096",
        ("per_channel",),
        (Layer("llama3_8b_gate_up_m256", M=256, K=4096, N=28672, seed=3000, x_kind="silu_mul"),
         Layer("llama3_8b_down_m256", M=256, K=14336, N=4096, seed=3001, x_kind="silu_mul"))),
    "llama3_8b_prefill": Workload(
        "llama3_8b_prefill", "Llama-3-8B prefill, M=4096: o_proj K=4096 N=4096, gate_up K=4096 N=28672",
        ("g128", "per_channel"),
        # 1% of the 4096 activation channels (41) carry x20 values.
        (Layer("llama3_8b_o_proj_m4096", M=4096, K=4096, N=4096, seed=4000,
               x_outliers=41, x_outlier_scale=20.0),
         Layer("llama3_8b_gate_up_m4096", M=4096, K=4096, N=28672, seed=4001,
               x_outliers=41, x_outlier_scale=20.0))),
    "qwen15_72b_m16": Workload("qwen15_72b_m16", "Qwen1.5-72B layers at M=16", ("g128", "per_channel"),
                               _qwen_layers(16)),
    "qwen15_72b_m128": Workload("qwen15_72b_m128", "Qwen1.5-72B layers at M=128", ("g128", "per_channel"),
                                _qwen_layers(128)),
    "qwen15_72b_m1024": Workload("qwen15_72b_m1024", "Qwen1.5-72B layers at M=1024",
                                 ("g128", "per_channel"), _qwen_layers(1024)),
}


def generate(layer: Layer, device: str = "cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """Return (x [M,K] fp16, w [N,K] fp16) for `layer`, drawn on the CPU."""
    g = torch.Generator(device="cpu")
    g.manual_seed(layer.seed)
    w = torch.randn(layer.N, layer.K, generator=g, dtype=torch.float32)
    w.mul_(layer.w_sigma)
    if layer.w_outliers:
        idx = torch.randperm(layer.K, generator=g)[: layer.w_outliers]
        w[:, idx] *= layer.w_outlier_scale
    w16 = w.to(torch.float16)
    del w
    rows = layer.rows_drawn
    if layer.x_kind == "normal":
        x = torch.randn(rows, layer.K, generator=g, dtype=torch.float32)
    elif layer.x_kind == "silu_mul":
        a = torch.randn(rows, layer.K, generator=g, dtype=torch.float32)
        b = torch.randn(rows, layer.K, generator=g, dtype=torch.float32)
        x = torch.nn.functional.silu(a) * b
    else:
        raise ValueError(layer.x_kind)
    if layer.x_outliers:
        idx = torch.randperm(layer.K, generator=g)[: layer.x_outliers]
        x[:, idx] *= layer.x_outlier_scale
    x16 = x[: layer.M].to(torch.float16).contiguous()
    if device != "cpu":
        return x16.to(device), w16.to(device)
    return x16, w16


def random_fp16(shape, seed: int, scale: float = 1.0) -> torch.Tensor:
    """Plain N(0, scale) FP16 tensor for small parity cases."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (torch.randn(*shape, generator=g, dtype=torch.float32) * scale).to(torch.float16)


def all_layers() -> List[Layer]:
    out = []
    for wl in WORKLOADS.values():
        out.extend(wl.layers)
    return out
