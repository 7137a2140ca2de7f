"""A packed weight written as a checkpoint (64-byte header, blob, scales) and
read back gives the same blob, scales and GEMM outputs, in every format."""
import pytest
import torch

import quantized_gemm_qoq_amd as qoq
from quantized_gemm_qoq_amd import workloads

from gpu_util import DEV

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


@pytest.mark.parametrize("mode", ["g128", "per_channel", "w8a8"])
def test_checkpoint_round_trip(mode, tmp_path):
    N, K, M = 272, 640, 33
    pw = qoq.PackedWeight(mode, workloads.random_fp16((N, K), 500, 0.02).to(DEV))
    path = str(tmp_path / f"{mode}.qpk")
    pw.save(path)
    back = qoq.PackedWeight.load(path, mode, N, K, DEV)
    assert torch.equal(back.blob, pw.blob)
    assert torch.equal(back.s_c.view(torch.int16), pw.s_c.view(torch.int16))
    x = workloads.random_fp16((M, K), 501, 1.0).to(DEV)
    assert torch.equal(back.forward(x), pw.forward(x))
