"""GPU parity of the RMSNorm producer of a GEMM input (y = f16((x * r) * gamma),
r = 1 / sqrt(f32(f64(S) / K) + eps) from the exact sum of squares S, then
per-token INT8 quantization) against the CPU oracle, through the C ABI.
Everything here is bit-exact: y, the packed INT8 codes, the scales and the row
sums."""
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


def _wide_rows(rng, M, K):
    """Rows mixing FP16 subnormals, ordinary values, zeros and values near
    65504, so the exact sum of squares needs all of its 80-odd bits and its
    rounding to fp64 is exercised."""
    e = rng.integers(-24, 16, size=(M, K)).astype(np.float32)
    x = np.exp2(e) * rng.uniform(1.0, 1.99, size=(M, K)).astype(np.float32)
    x *= np.where(rng.random((M, K)) < 0.5, -1.0, 1.0).astype(np.float32)
    x[rng.random((M, K)) < 0.1] = 0.0
    return np.clip(x, -65504, 65504).astype(np.float16)


def _check(x16, gamma16, eps, want_rowsum=True, want_y=True):
    xb, gb = x16.view(np.uint16), gamma16.view(np.uint16)
    y_w, xq_w, sx_w, rs_w = oracle.rmsnorm_quantize_act(xb, gb, eps)
    M, K = x16.shape
    y = torch.empty((M, K), dtype=torch.float16, device=DEV) if want_y else None
    xq, s_x, rs = qoq.qoq_rmsnorm_quantize_act(f16_dev(xb), f16_dev(gb), eps,
                                                want_rowsum=want_rowsum, y=y)
    torch.cuda.synchronize()
    if want_y:
        np.testing.assert_array_equal(host_bits(y), y_w)
    np.testing.assert_array_equal(host(xq), oracle.pack_act(xq_w))
    np.testing.assert_array_equal(host_bits(s_x), sx_w)
    if want_rowsum:
        np.testing.assert_array_equal(host(rs), rs_w)
    else:
        assert rs is None


@pytest.mark.parametrize("M,K", [(1, 128), (7, 384), (64, 4096), (33, 8192), (5, 14336),
                                 (16, 24576), (3, 32768)])
def test_rmsnorm_producer_shapes(M, K):
    """Each row size of the kernel (256 or 1024 threads, one or two 16-input
    runs each), ragged row counts, ordinary activations with outlier channels,
    and special rows: all zero (y = 0), one input, a constant row."""
    rng = np.random.default_rng(1000 + K + M)
    x = workloads.random_fp16((M, K), 1001 + M, 1.0).numpy()
    x[:, rng.choice(K, size=max(1, K // 100), replace=False)] *= np.float16(20.0)
    if M > 1:
        x[1] = 0
    if M > 2:
        x[2] = 0
        x[2, K // 3] = np.float16(-7.0)
    if M > 3:
        x[3] = np.float16(0.125)
    gamma = rng.uniform(0.2, 2.0, size=K).astype(np.float16)
    print(f"rmsnorm producer M={M} K={K}", flush=True)
    _check(x, gamma, 1e-5)


@pytest.mark.parametrize("eps", [1e-5, 1e-6, 1e-30, 0.5])
def test_rmsnorm_wide_range_rows(eps):
    """Rows spanning the whole FP16 range: the 128-bit sum, its rounding to
    fp64 and the rest of the scale are bit-identical to the oracle's."""
    rng = np.random.default_rng(1100)
    x = _wide_rows(rng, 96, 1024)
    gamma = rng.uniform(0.5, 1.5, size=1024).astype(np.float16)
    print(f"rmsnorm wide rows eps={eps}", flush=True)
    _check(x, gamma, eps)


def test_rmsnorm_many_scales():
    """4096 short rows: 4096 different sums of squares, each rounded through
    the fp64 mean, fp32 square root and reciprocal exactly as the oracle does."""
    rng = np.random.default_rng(1200)
    x = (rng.standard_normal((4096, 128)) * np.exp2(rng.integers(-6, 7, size=(4096, 1)))).astype(np.float16)
    gamma = rng.uniform(0.5, 1.5, size=128).astype(np.float16)
    print("rmsnorm 4096 rows", flush=True)
    _check(x, gamma, 1e-6)


def test_rmsnorm_optional_outputs_and_empty():
    rng = np.random.default_rng(1300)
    x = workloads.random_fp16((9, 640), 1301, 2.0).numpy()
    gamma = rng.uniform(0.5, 1.5, size=640).astype(np.float16)
    _check(x, gamma, 1e-5, want_rowsum=False, want_y=False)
    _check(x, gamma, 1e-5, want_rowsum=True, want_y=False)
    g = f16_dev(gamma.view(np.uint16))
    xq, s_x, rs = qoq.qoq_rmsnorm_quantize_act(torch.empty((0, 640), dtype=torch.float16, device=DEV),
                                                g, 1e-5)
    assert xq.numel() == 0


@pytest.mark.parametrize("mode", [qoq.MODE_G128, qoq.MODE_PER_CHANNEL])
def test_rmsnorm_then_qkv_gemm(mode):
    """The attention input on the GPU: RMSNorm producer -> qkv GEMM, against the
    oracle running the same chain on the same x (the codes and accumulators
    bit-exactly, Y within tolerance)."""
    M, D, N = 40, 1024, 1536
    rng = np.random.default_rng(1400)
    x = workloads.random_fp16((M, D), 1401, 1.0).numpy()
    gamma = rng.uniform(0.5, 1.5, size=D).astype(np.float16)
    w = workloads.random_fp16((N, D), 1402, 0.05).numpy().view(np.uint16)
    pw = qoq.PackedWeight(mode, f16_dev(w))
    xq, s_x, rs = qoq.qoq_rmsnorm_quantize_act(f16_dev(x.view(np.uint16)), f16_dev(gamma.view(np.uint16)),
                                                1e-5, want_rowsum=mode == qoq.MODE_PER_CHANNEL)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y = qoq.qoq_w4a8_gemm(mode, xq, s_x, rs, pw.blob, pw.s_c, N, acc_out=acc)
    torch.cuda.synchronize()
    print(f"rmsnorm -> qkv mode={mode}", flush=True)
    _, oxq, osx, _ = oracle.rmsnorm_quantize_act(x.view(np.uint16), gamma.view(np.uint16), 1e-5)
    np.testing.assert_array_equal(host(xq), oracle.pack_act(oxq))
    wq = oracle.quantize_weights(mode, w)
    acc_w = oracle.gemm(mode, oxq, wq["q"], wq["s_g"], wq["z"])
    np.testing.assert_array_equal(host(acc), acc_w)
    assert_y_close(host_bits(y), oracle.epilogue(acc_w, osx, wq["s_c"]), "qkv")
