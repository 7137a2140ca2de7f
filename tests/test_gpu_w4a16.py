"""GPU parity of the W4A16 sibling (FP16 activations, the same QoQ 4-bit
weights) against the CPU oracle, through the C ABI.

The GPU accumulates exact products in FP32 in an order of its own, so the
output is compared with the oracle's fp64 value under the bound that this
arithmetic admits, element by element:
    |y - Y| <= s_c * (K - 1) * 2^-24 * sum_k |x * W8^|   (FP32 accumulation)
             + 2^-23 * |Y|                              (FP32 product by s_c)
             + one FP16 ulp of |Y|                      (final rounding)
and, over the whole output, within 1e-3 * max|Y|. The FP16 output must also be
exactly the rounded product of the FP32 accumulator (acc_out) and s_c.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_qoq_amd as qoq
from quantized_gemm_qoq_amd import workloads

from gpu_util import DEV, f16_dev, host, host_bits, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

G128, PC = qoq.MODE_G128, qoq.MODE_PER_CHANNEL


def _rand_bits(shape, seed, scale):
    return workloads.random_fp16(shape, seed, scale).numpy().view(np.uint16)


def assert_w4a16_close(y_bits, y_ref, absum, K, what=""):
    yg = np.asarray(y_bits, np.uint16).view(np.float16).astype(np.float64)
    ref = np.asarray(y_ref, np.float64)
    over = np.abs(ref) >= 65504.0 * (1 + 2.0**-12)
    assert np.all(np.isinf(yg[over])), what
    yg, ref, ab = yg[~over], ref[~over], np.asarray(absum, np.float64)[~over]
    err = np.abs(yg - ref)
    ulp = np.maximum(np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64), 2.0**-24)
    bound = (K - 1) * 2.0**-24 * ab + 2.0**-23 * np.abs(ref) + ulp
    bad = err > bound
    assert not bad.any(), (what, float((err / bound).max()), int(bad.sum()))
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    assert err.max(initial=0.0) <= 1e-3 * scale + 1e-30, (what, err.max(), scale)


def _epilogue_consistent(y_bits, acc, s_c_bits):
    sc = np.asarray(s_c_bits, np.uint16).view(np.float16).astype(np.float32)
    want = (acc.astype(np.float32) * sc[None, :]).astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(y_bits, want)


SHAPES = [
    (1, 16, 128), (8, 256, 512), (17, 48, 384), (33, 96, 1152), (64, 160, 256),
    (9, 32, 128 * 21), (30, 48, 128 * 67),
    (65, 32, 640), (100, 272, 256), (129, 512, 1024), (257, 80, 128), (520, 272, 640),
    (3, 16, 132096),
]


@pytest.mark.parametrize("mode", [G128, PC])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w4a16_gemm_against_oracle(mode, M, N, K):
    xb = _rand_bits((M, K), 240 + M + K, 1.0)
    if M > 1:
        xb[1] = 0  # a zero row
    if M > 2:
        xb[2, 3] = np.float16(-300.0).view(np.uint16)  # an outlier activation
    wb = _rand_bits((N, K), 250 + N + K, 0.02 if K < 65536 else 0.002)
    if N > 1:
        wb[1] = 0  # a zero channel: s_c = 0
    wq = oracle.quantize_weights(mode, wb)
    y_want, absum = oracle.gemm_w4a16(mode, xb, wq["s_c"], wq["q"], wq["s_g"], wq["z"])
    blob = oracle.pack(mode, wq["q"], wq["s_g"], wq["z"])
    print(f"w4a16 gemm mode={mode} M={M} N={N} K={K}", flush=True)
    d_sc = to_dev(wq["s_c"], torch.float16)
    acc = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y_acc = qoq.qoq_w4a16_gemm(mode, f16_dev(xb), to_dev(blob), d_sc, N, acc_out=acc)
    y = qoq.qoq_w4a16_gemm(mode, f16_dev(xb), to_dev(blob), d_sc, N)
    torch.cuda.synchronize()
    assert_w4a16_close(host_bits(y), y_want, absum, K, f"mode {mode}")
    np.testing.assert_array_equal(host_bits(y_acc), host_bits(y))
    _epilogue_consistent(host_bits(y), host(acc), wq["s_c"])


@pytest.mark.parametrize("mode", [G128, PC])
def test_w4a16_full_path_and_empty(mode):
    M, N, K = 40, 272, 768
    xb = _rand_bits((M, K), 261, 1.0)
    wb = _rand_bits((N, K), 262, 0.02)
    res = oracle.forward_w4a16(mode, xb, wb)
    pw = qoq.PackedWeight(mode, f16_dev(wb))
    y = pw.forward_fp16(f16_dev(xb))
    e = pw.forward_fp16(torch.empty((0, K), dtype=torch.float16, device=DEV))
    z = pw.forward_fp16(torch.zeros((5, K), dtype=torch.float16, device=DEV))
    torch.cuda.synchronize()
    assert_w4a16_close(host_bits(y), res["y"], res["absum"], K, "end to end")
    assert e.shape == (0, N)
    assert torch.all(z == 0)


def test_w4a16_is_deterministic():
    M, N, K = 48, 512, 2048
    pw = qoq.PackedWeight(G128, f16_dev(_rand_bits((N, K), 271, 0.02)))
    x = f16_dev(_rand_bits((M, K), 272, 1.0))
    y0 = pw.forward_fp16(x).clone()
    for _ in range(3):
        assert torch.equal(pw.forward_fp16(x), y0)


FULL = [
    (workloads.WORKLOADS["llama3_8b_qkv_decode"].layers[0], "g128"),
    (workloads.WORKLOADS["llama3_8b_qkv_decode"].layers[0], "per_channel"),
    (workloads.WORKLOADS["qwen15_72b_m16"].layers[3], "g128"),
    (workloads.WORKLOADS["llama3_8b_mlp_m256"].layers[1], "per_channel"),
    (workloads.WORKLOADS["llama3_8b_prefill"].layers[0], "g128"),
]


@pytest.mark.parametrize("layer,mode", FULL, ids=lambda v: v if isinstance(v, str) else v.name)
def test_w4a16_layer_parity(layer, mode):
    M, N, K = layer.M, layer.N, layer.K
    mode_id = qoq.MODES[mode]
    print(f"w4a16 layer {layer.name} {mode} M={M} K={K} N={N}", flush=True)
    x16, w16 = workloads.generate(layer)
    xb, wb = x16.numpy().view(np.uint16), w16.numpy().view(np.uint16)
    pw = qoq.PackedWeight(mode_id, w16.to(DEV))
    x = x16.to(DEV)
    y = pw.forward_fp16(x)
    acc = torch.empty((M, N), dtype=torch.float32, device=DEV)
    qoq.qoq_w4a16_gemm(mode_id, x, pw.blob, pw.s_c, N, acc_out=acc)
    torch.cuda.synchronize()
    wq = oracle.quantize_weights(mode_id, wb)
    np.testing.assert_array_equal(host_bits(pw.s_c), wq["s_c"])
    y_want, absum = oracle.gemm_w4a16_matmul(mode_id, xb, wq["s_c"], wq["q"], wq["s_g"], wq["z"])
    y_h = host_bits(y)
    assert_w4a16_close(y_h, y_want, absum, K, layer.name)
    _epilogue_consistent(y_h, host(acc), wq["s_c"])
