"""qoq_w4a8_gemm_noalloc, called through the C ABI, gives the same INT32
accumulators and FP16 outputs as qoq_w4a8_gemm with a caller workspace, on two
calls in a row (the second smaller, so it reuses scratch the first left
behind), for shapes whose plan uses the scratch (split K) and shapes whose
plan does not; no plan needs more scratch than the fixed array."""
import ctypes

import pytest
import torch

import quantized_gemm_qoq_amd as qoq
from quantized_gemm_qoq_amd import workloads

from gpu_util import DEV

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

LIMIT = 32 * 1024 * 1024


def _inputs(M, K, N, mode, seed):
    pw = qoq.PackedWeight(mode, workloads.random_fp16((N, K), seed, 0.02).to(DEV))
    xq, s_x, rowsum = qoq.qoq_quantize_act(workloads.random_fp16((M, K), seed + 1, 1.0).to(DEV))
    return pw, xq, s_x, rowsum


def _noalloc(mode, pw, xq, s_x, rowsum, M, N, K, y, acc):
    lib = qoq.load_library()
    return lib.qoq_w4a8_gemm_noalloc(qoq.MODES[mode], qoq._ptr(xq), qoq._ptr(s_x), qoq._ptr(rowsum),
                                     qoq._ptr(pw.blob), qoq._ptr(pw.s_c), M, N, K, qoq._ptr(y),
                                     qoq._ptr(acc), qoq._stream(xq))


# (first call, second smaller call): split-K plans (scratch used) and plans without.
PAIRS = [((128, 24576, 8192), (200, 1664, 272)),  # 32 MiB of partial sums, then a small split
         ((256, 4096, 2048), (130, 1024, 144)),
         ((64, 4096, 6144), (17, 384, 272)),       # decode plans: no scratch
         ((600, 1152, 528), (65, 512, 272))]


@pytest.mark.parametrize("mode", ["g128", "per_channel"])
@pytest.mark.parametrize("first,second", PAIRS, ids=lambda v: "x".join(map(str, v)))
def test_noalloc_matches_workspace_entry_point(mode, first, second):
    for i, (M, K, N) in enumerate((first, second)):
        need = qoq.qoq_gemm_workspace_bytes(mode, M, N, K)
        assert 0 <= need <= LIMIT
        pw, xq, s_x, rowsum = _inputs(M, K, N, mode, 300 + 10 * i + M)
        rs = rowsum if mode == "per_channel" else None
        ws = torch.zeros((max(need, 16),), dtype=torch.uint8, device=DEV)
        acc_ref = torch.empty((M, N), dtype=torch.int32, device=DEV)
        y_ref = qoq.qoq_w4a8_gemm(mode, xq, s_x, rs, pw.blob, pw.s_c, N, acc_out=acc_ref,
                                  workspace=ws if need else None, K=K)
        y = torch.full((M, N), 7.0, dtype=torch.float16, device=DEV)
        acc = torch.full((M, N), -1, dtype=torch.int32, device=DEV)
        assert _noalloc(mode, pw, xq, s_x, rs, M, N, K, y, acc) == 0
        y2 = torch.full((M, N), 7.0, dtype=torch.float16, device=DEV)
        assert _noalloc(mode, pw, xq, s_x, rs, M, N, K, y2, None) == 0  # fast path, no acc_out
        torch.cuda.synchronize()
        assert torch.equal(acc, acc_ref), (M, K, N)
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (M, K, N)
        assert torch.equal(y2.view(torch.int16), y_ref.view(torch.int16)), (M, K, N)


def test_no_plan_needs_more_than_the_scratch():
    """Every split-K plan keeps S x (128 x 256 blocks) <= 256, so its partial
    sums never exceed 256 x 128 x 256 x 4 bytes = 32 MiB: the fixed scratch
    serves every shape (the refusal above the limit is a guard only)."""
    worst = 0
    for M in (65, 100, 128, 129, 200, 250, 256, 300, 384, 511, 512, 640, 1024):
        for N in (16, 272, 1024, 4096, 8192, 8208, 12288, 16384, 24576):
            for K in (256, 1024, 4096, 24576):
                for mode in ("g128", "per_channel"):
                    worst = max(worst, qoq.qoq_gemm_workspace_bytes(mode, M, N, K))
    assert 0 < worst <= LIMIT


def test_noalloc_empty_and_invalid_calls_launch_nothing():
    lib = qoq.load_library()
    assert lib.qoq_w4a8_gemm_noalloc(0, None, None, None, None, None, 0, 16, 128, None, None, None) == 0
    assert lib.qoq_w4a8_gemm_noalloc(0, None, None, None, None, None, 4, 15, 128, None, None, None) == 2
    assert lib.qoq_w4a8_gemm_noalloc(7, None, None, None, None, None, 4, 16, 128, None, None, None) == 4
    assert lib.qoq_w4a8_gemm_noalloc(0, None, None, None, None, None, 4, 16, 128, None, None, None) == 1
