"""GPU parity of the W8A8 sibling against the CPU oracle, through the C ABI.

Bit-exact for the INT8 weights, their scales, the packed blob and the INT32
accumulators; the FP16 output within 1e-3 * max|Y| of the oracle's exact value
and within one FP16 ulp element by element. The GEMM shapes run every kernel of
the plan (streaming decode kernel, split-K and unsplit tiled kernels, the
wide-wave kernel) with ragged rows, channels and group counts.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_qoq_amd as qoq
from quantized_gemm_qoq_amd import workloads

from gpu_util import DEV, assert_y_close, f16_dev, host, host_bits, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def _rand_bits(shape, seed, scale):
    return workloads.random_fp16(shape, seed, scale).numpy().view(np.uint16)


def _edge_rows(w_bits):
    w = w_bits.copy()
    N, K = w.shape
    if N > 1:
        w[1] = 0  # all zero: scale 0, codes 0
    if N > 2:
        w[2] = np.float16(-0.75).view(np.uint16)  # constant: every code -127
    if N > 3:
        w[3] = 0
        w[3, K // 2] = np.float16(2.0).view(np.uint16)  # single element
    if N > 4:
        w[4] = 0
        w[4, 9] = 0x0005  # subnormal maximum: the scale underflows to 0
    return w


@pytest.mark.parametrize("N,K", [(16, 128), (48, 640), (256, 4096), (32, 132096)])
def test_w8a8_quantize_weights(N, K):
    wb = _edge_rows(_rand_bits((N, K), 120 + N, 0.02))
    if N > 8:
        wb[8, 7] = np.float16(0.9).view(np.uint16)  # an outlier
    print(f"w8a8 quantize_weights N={N} K={K}", flush=True)
    s_want, q_want = oracle.quantize_weights_w8(wb)
    q, s_c = qoq.qoq_w8a8_quantize_weights(f16_dev(wb))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(s_c), s_want)
    np.testing.assert_array_equal(host(q), q_want)


def test_w8a8_scales_exhaustive_over_fp16_row_max():
    """Every positive finite FP16 value as a row's largest magnitude: the scale
    max/127 and the codes of the row match the oracle bit for bit."""
    vals = np.arange(1, 0x7C00, dtype=np.uint16)
    rows = (vals.size + 15) // 16 * 16
    w = np.zeros((rows, 128), np.uint16)
    w[: vals.size, 0] = vals
    w[: vals.size, 1] = vals | 0x8000
    w[: vals.size, 2] = vals - 1
    w[: vals.size, 3] = vals >> 1
    print(f"w8a8 exhaustive scales over {vals.size} rows", flush=True)
    s_want, q_want = oracle.quantize_weights_w8(w)
    q, s_c = qoq.qoq_w8a8_quantize_weights(f16_dev(w))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(s_c), s_want)
    np.testing.assert_array_equal(host(q), q_want)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 640), (96, 2176)])
def test_w8a8_pack(N, K):
    rng = np.random.default_rng(N + K)
    q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    print(f"w8a8 pack N={N} K={K}", flush=True)
    blob = qoq.qoq_w8a8_pack_weights(to_dev(q))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(blob), oracle.pack_w8(q))


GEMM_SHAPES = [
    (1, 16, 128), (8, 256, 512), (17, 48, 384), (64, 96, 1152), (100, 160, 256),
    (129, 32, 640), (257, 80, 128), (512, 512, 1024), (520, 272, 640), (3, 16, 132096),
    (9, 32, 128 * 21), (30, 48, 128 * 67), (48, 64, 128 * 70),
    (200, 272, 128 * 13),
    (600, 528, 128 * 9), (700, 400, 128 * 10), (200, 16400, 128 * 3), (1024, 8208, 128 * 13),
    # the large-block persistent kernel: one, two and 1.5 rounds of 256 x 256 blocks
    (4000, 4000, 128 * 8), (4000, 8000, 128 * 4), (1000, 24560, 128 * 4),
]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_w8a8_gemm_against_oracle(M, N, K):
    xb = _rand_bits((M, K), 140 + M + K, 1.0)
    wb = _edge_rows(_rand_bits((N, K), 150 + N + K, 0.02 if K < 65536 else 0.002))
    xq, s_x, _ = oracle.quantize_act(xb)
    s_c, q = oracle.quantize_weights_w8(wb)
    acc_want = oracle.gemm_w8(xq, q)
    y_want = oracle.epilogue(acc_want, s_x, s_c)
    print(f"w8a8 gemm M={M} N={N} K={K}", flush=True)
    d_xq, d_sx = to_dev(oracle.pack_act(xq)), to_dev(s_x, torch.float16)
    d_blob, d_sc = to_dev(oracle.pack_w8(q)), to_dev(s_c, torch.float16)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y_acc = qoq.qoq_w8a8_gemm(d_xq, d_sx, d_blob, d_sc, N, acc_out=acc)
    y = qoq.qoq_w8a8_gemm(d_xq, d_sx, d_blob, d_sc, N)
    y_ws = qoq.qoq_w8a8_gemm(d_xq, d_sx, d_blob, d_sc, N, workspace=None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(acc), acc_want)
    assert_y_close(host_bits(y), y_want, "fast path")
    np.testing.assert_array_equal(host_bits(y_acc), host_bits(y))
    np.testing.assert_array_equal(host_bits(y_ws), host_bits(y))


def test_w8a8_full_path_and_empty():
    M, N, K = 33, 272, 768
    xb = _rand_bits((M, K), 161, 1.0)
    wb = _rand_bits((N, K), 162, 0.02)
    res = oracle.forward_w8(xb, wb)
    pw = qoq.PackedWeight(qoq.W8A8, f16_dev(wb))
    y = pw.forward(f16_dev(xb))
    e = pw.forward(torch.empty((0, K), dtype=torch.float16, device=DEV))
    z = pw.forward(torch.zeros((5, K), dtype=torch.float16, device=DEV))
    torch.cuda.synchronize()
    assert_y_close(host_bits(y), res["y"], "end to end")
    assert e.shape == (0, N)
    assert torch.all(z == 0)


# The decode and prefill layers the format comparison times, at full size.
FULL_LAYERS = [
    workloads.WORKLOADS["llama3_8b_qkv_decode"].layers[0],
    workloads.WORKLOADS["qwen15_72b_m16"].layers[3],
    workloads.WORKLOADS["llama3_8b_mlp_m256"].layers[1],
    workloads.WORKLOADS["llama3_8b_prefill"].layers[0],
]


@pytest.mark.parametrize("layer", FULL_LAYERS, ids=lambda l: l.name)
def test_w8a8_layer_parity(layer):
    M, N, K = layer.M, layer.N, layer.K
    print(f"w8a8 layer {layer.name} M={M} K={K} N={N}", flush=True)
    x16, w16 = workloads.generate(layer)
    xb, wb = x16.numpy().view(np.uint16), w16.numpy().view(np.uint16)
    pw = qoq.PackedWeight(qoq.W8A8, w16.to(DEV))
    xq, s_x, _ = qoq.qoq_quantize_act(x16.to(DEV), want_rowsum=False)
    y = qoq.qoq_w8a8_gemm(xq, s_x, pw.blob, pw.s_c, N)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    qoq.qoq_w8a8_gemm(xq, s_x, pw.blob, pw.s_c, N, acc_out=acc)
    torch.cuda.synchronize()
    oxq, osx, _ = oracle.quantize_act(xb)
    s_c, q = oracle.quantize_weights_w8(wb)
    np.testing.assert_array_equal(host_bits(pw.s_c), s_c)
    np.testing.assert_array_equal(host(pw.blob), oracle.pack_w8(q))
    acc_want = oracle.gemm_w8_matmul(oxq, q)
    acc_h = host(acc)
    np.testing.assert_array_equal(acc_h, acc_want)
    y_h = host_bits(y)
    assert_y_close(y_h, oracle.epilogue(acc_want, osx, s_c), layer.name)
    sx = osx.view(np.float16).astype(np.float32)
    sc = s_c.view(np.float16).astype(np.float32)
    y_from_acc = ((acc_h.astype(np.float32) * sx[:, None]) * sc[None, :]).astype(np.float16)
    np.testing.assert_array_equal(y_h, y_from_acc.view(np.uint16))
