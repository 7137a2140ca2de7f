"""GPU parity of the fused producer of the down projection's input
(h = f16(SiLU(gate) * up), then per-token INT8 quantization) against the CPU
oracle, through the C ABI. Everything here is bit-exact: h, the packed INT8
codes, the scales and the row sums."""
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


def _run(gu_bits, want_rowsum=True, want_h=True):
    M, I2 = gu_bits.shape
    h = torch.empty((M, I2 // 2), dtype=torch.float16, device=DEV) if want_h else None
    xq, s_x, rs = qoq.qoq_silu_mul_quantize_act(f16_dev(gu_bits), want_rowsum=want_rowsum, h=h)
    torch.cuda.synchronize()
    return xq, s_x, rs, h


def _check(gu_bits, want_rowsum=True, want_h=True):
    h_w, xq_w, sx_w, rs_w = oracle.silu_mul_quantize_act(gu_bits)
    xq, s_x, rs, h = _run(gu_bits, want_rowsum, want_h)
    if want_h:
        np.testing.assert_array_equal(host_bits(h), h_w)
    np.testing.assert_array_equal(host(xq), oracle.pack_act(xq_w))
    np.testing.assert_array_equal(host_bits(s_x), sx_w)
    if want_rowsum:
        np.testing.assert_array_equal(host(rs), rs_w)
    else:
        assert rs is None


def test_every_fp16_gate_value():
    """Every finite FP16 value as the gate (up = 1, then up = -0.75): h and the
    codes match the oracle bit for bit, which checks the exponential, the
    division and the FP16 rounding on every input they can see."""
    vals = np.concatenate([np.arange(0, 0x7C00), np.arange(0x8000, 0xFC00)]).astype(np.uint16)
    I = 1024
    rows = (vals.size + I - 1) // I
    g = np.zeros(rows * I, np.uint16)
    g[: vals.size] = vals
    g = g.reshape(rows, I)
    print(f"fused producer: {vals.size} gate values in {rows} rows", flush=True)
    for up in (1.0, -0.75):
        u = np.full((rows, I), np.float16(up).view(np.uint16), np.uint16)
        _check(np.concatenate([g, u], axis=1))


@pytest.mark.parametrize("M,I", [(1, 128), (7, 384), (64, 4096), (33, 14336), (5, 24576),
                                 (3, 32768 + 128), (2, 132096)])
def test_fused_producer_shapes(M, I):
    """Each row size of the register-resident kernel, the two-pass kernel above
    32768, and the largest I; ragged row counts."""
    gate = workloads.random_fp16((M, I), 300 + M, 3.0).numpy()
    up = workloads.random_fp16((M, I), 301 + M, 1.0).numpy()
    if M > 1:
        gate[1] = 0  # h = 0: zero scale, zero codes
    if M > 2:
        gate[2, 5] = np.float16(-90.0)  # exp above its cut-off
        gate[2, 6] = np.float16(95.0)   # exp below its cut-off
    print(f"fused producer M={M} I={I}", flush=True)
    _check(np.concatenate([gate, up], axis=1).view(np.uint16))


@pytest.mark.parametrize("M,I", [(1, 24576), (16, 24576), (32, 14336), (17, 12288), (3, 12416),
                                 (5, 132096)])
def test_split_rows_match_one_pass_and_oracle(M, I):
    """Few rows: the split path (several workgroups per row, two passes) gives
    the oracle's outputs bit for bit, as do the one-pass kernels through both
    entry points; the workspace needs no initialisation."""
    import ctypes
    gate = workloads.random_fp16((M, I), 330 + M, 3.0).numpy()
    up = workloads.random_fp16((M, I), 331 + M, 1.0).numpy()
    gu = np.concatenate([gate, up], axis=1).view(np.uint16)
    print(f"fused producer split M={M} I={I}", flush=True)
    _check(gu)  # the binding's default: split when the shape gains from it
    lib = qoq.load_library()
    need = lib.qoq_silu_mul_workspace_bytes(M, I)
    assert need > 0
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
    h_w, xq_w, sx_w, rs_w = oracle.silu_mul_quantize_act(gu)
    d_gu = f16_dev(gu)
    for how in ("split", "one-pass", "plain"):
        h = torch.empty((M, I), dtype=torch.float16, device=DEV)
        xq = torch.empty((qoq.qoq_act_bytes(M, I),), dtype=torch.int8, device=DEV)
        s_x = torch.empty((M,), dtype=torch.float16, device=DEV)
        rs = torch.full((M,), 12345, dtype=torch.int32, device=DEV)
        ptr = lambda t: ctypes.c_void_p(t.data_ptr())
        if how == "plain":
            st = lib.qoq_silu_mul_quantize_act(ptr(d_gu), M, I, ptr(xq), ptr(s_x), ptr(rs), ptr(h), None)
        else:
            w = ws if how == "split" else None
            st = lib.qoq_silu_mul_quantize_act_ws(ptr(d_gu), M, I, ptr(xq), ptr(s_x), ptr(rs), ptr(h),
                                                  None if w is None else ptr(w), 0 if w is None else need,
                                                  None)
        assert st == 0, how
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(h), h_w, err_msg=how)
        np.testing.assert_array_equal(host(xq), oracle.pack_act(xq_w), err_msg=how)
        np.testing.assert_array_equal(host_bits(s_x), sx_w, err_msg=how)
        np.testing.assert_array_equal(host(rs), rs_w, err_msg=how)
    # again on the same workspace (its row tallies left from the call above),
    # with fewer rows and no h output
    M2 = max(1, M // 2)
    gu2 = np.ascontiguousarray(gu[:M2])
    _, xq_w2, sx_w2, rs_w2 = oracle.silu_mul_quantize_act(gu2)
    xq = torch.empty((qoq.qoq_act_bytes(M2, I),), dtype=torch.int8, device=DEV)
    s_x = torch.empty((M2,), dtype=torch.float16, device=DEV)
    rs = torch.full((M2,), 12345, dtype=torch.int32, device=DEV)
    need2 = lib.qoq_silu_mul_workspace_bytes(M2, I)
    st = lib.qoq_silu_mul_quantize_act_ws(ptr(f16_dev(gu2)), M2, I, ptr(xq), ptr(s_x), ptr(rs), None,
                                          ptr(ws) if need2 else None, need2, None)
    assert st == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(xq), oracle.pack_act(xq_w2))
    np.testing.assert_array_equal(host_bits(s_x), sx_w2)
    np.testing.assert_array_equal(host(rs), rs_w2)


def test_fused_producer_optional_outputs():
    gu = workloads.random_fp16((9, 2 * 640), 310, 2.0).numpy().view(np.uint16)
    _check(gu, want_rowsum=False, want_h=False)
    _check(gu, want_rowsum=True, want_h=False)
    xq, s_x, rs = qoq.qoq_silu_mul_quantize_act(torch.empty((0, 256), dtype=torch.float16,
                                                            device=DEV))
    assert xq.numel() == 0


@pytest.mark.parametrize("mode", [qoq.MODE_G128, qoq.MODE_PER_CHANNEL])
def test_mlp_chain_gate_up_then_down(mode):
    """The MLP on the GPU: gate_up GEMM -> fused producer -> down GEMM, against
    the oracle running the same chain on the GPU's gate_up output (the first
    GEMM is checked on its own within tolerance, the rest bit-exactly on
    identical inputs)."""
    M, D, I = 40, 512, 768
    x = workloads.random_fp16((M, D), 320, 1.0).numpy().view(np.uint16)
    w_gu = workloads.random_fp16((2 * I, D), 321, 0.05).numpy().view(np.uint16)
    w_dn = workloads.random_fp16((D, I), 322, 0.05).numpy().view(np.uint16)
    pw_gu = qoq.PackedWeight(mode, f16_dev(w_gu))
    pw_dn = qoq.PackedWeight(mode, f16_dev(w_dn))
    gu = pw_gu.forward(f16_dev(x))
    xq, s_x, rs = qoq.qoq_silu_mul_quantize_act(gu, want_rowsum=mode == qoq.MODE_PER_CHANNEL)
    acc = torch.empty((M, D), dtype=torch.int32, device=DEV)
    y = qoq.qoq_w4a8_gemm(mode, xq, s_x, rs, pw_dn.blob, pw_dn.s_c, D, acc_out=acc)
    torch.cuda.synchronize()
    print(f"mlp chain mode={mode}", flush=True)
    ref_gu = oracle.forward(mode, x, w_gu)
    assert_y_close(host_bits(gu), ref_gu["y"], "gate_up")
    gu_bits = host_bits(gu)
    _, oxq, osx, ors = oracle.silu_mul_quantize_act(gu_bits)
    np.testing.assert_array_equal(host(xq), oracle.pack_act(oxq))
    wq = oracle.quantize_weights(mode, w_dn)
    acc_w = oracle.gemm(mode, oxq, wq["q"], wq["s_g"], wq["z"])
    np.testing.assert_array_equal(host(acc), acc_w)
    assert_y_close(host_bits(y), oracle.epilogue(acc_w, osx, wq["s_c"]), "down")
