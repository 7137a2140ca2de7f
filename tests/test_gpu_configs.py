"""GPU parity at the benchmark's full sizes: every layer of every workload, in
both modes where the workload names both.

The weights, the blob, the INT8 activations and the row sums are compared with
the oracle bit-exactly at full size. The GEMM is contracted in full on the host
(the oracle's library-product form, pinned to its C loops on the CPU) and every
INT32 accumulator of the GPU is compared with it; every FP16 output of the fast
path that the benchmark times (no accumulator output) is checked against the
oracle's exact rescale, and equals the rescale of the GPU's own accumulators.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_qoq_amd as qoq
from quantized_gemm_qoq_amd import workloads

from gpu_util import assert_y_close, host, host_bits

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


CASES = []
for wl in workloads.WORKLOADS.values():
    for layer in wl.layers:
        for mode in wl.modes:
            CASES.append(pytest.param(layer, mode, id=f"{layer.name}-{mode}"))


@pytest.mark.parametrize("layer,mode", CASES)
def test_layer_parity(layer, mode):
    mode_id = qoq.MODES[mode]
    print(f"layer {layer.name} mode {mode} M={layer.M} K={layer.K} N={layer.N}", flush=True)
    x16, w16 = workloads.generate(layer)
    xb = x16.numpy().view(np.uint16)
    wb = w16.numpy().view(np.uint16)
    dx, dw = x16.to("cuda:0"), w16.to("cuda:0")

    # GPU: the whole path, as the benchmark runs it.
    q, s_c, s_g, z = qoq.qoq_quantize_weights(mode_id, dw)
    blob = qoq.qoq_pack_weights(mode_id, q, s_g, z)
    del q, s_g
    xq, s_x, rowsum = qoq.qoq_quantize_act(dx)
    y = qoq.qoq_w4a8_gemm(mode_id, xq, s_x, rowsum if mode_id == qoq.MODE_PER_CHANNEL else None,
                          blob, s_c, layer.N)
    torch.cuda.synchronize()

    # Oracle: quantizers and pack in full.
    oxq, osx, ors = oracle.quantize_act(xb)
    np.testing.assert_array_equal(host(xq), oracle.pack_act(oxq))
    np.testing.assert_array_equal(host_bits(s_x), osx)
    np.testing.assert_array_equal(host(rowsum), ors)
    wq = oracle.quantize_weights(mode_id, wb)
    np.testing.assert_array_equal(host_bits(s_c), wq["s_c"])
    oblob = oracle.pack(mode_id, wq["q"], wq["s_g"], wq["z"])
    np.testing.assert_array_equal(host(blob), oblob)
    del oblob

    M, N, K = layer.M, layer.N, layer.K
    acc_want = oracle.gemm_matmul(mode_id, oxq, wq["q"], wq["s_g"], wq["z"])
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    qoq.qoq_w4a8_gemm(mode_id, xq, s_x, rowsum, blob, s_c, N, acc_out=acc)
    torch.cuda.synchronize()
    acc_h = host(acc)
    np.testing.assert_array_equal(acc_h, acc_want)
    y_h = host_bits(y)
    assert_y_close(y_h, oracle.epilogue(acc_want, osx, wq["s_c"]), layer.name)
    # The fast path's Y is the rescaled accumulator at every element.
    sx = osx.view(np.float16).astype(np.float32)
    sc = wq["s_c"].view(np.float16).astype(np.float32)
    y_from_acc = ((acc_h.astype(np.float32) * sx[:, None]) * sc[None, :]).astype(np.float16)
    np.testing.assert_array_equal(y_h, y_from_acc.view(np.uint16))
