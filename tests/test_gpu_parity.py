"""GPU parity: every kernel of the path against the CPU oracle, through the C ABI.

Bit-exact for the integer and byte results (codes, scales, zeros, the packed
blob, INT8 activations, row sums and the INT32 accumulators); the FP16 output
within 1e-3 * max|Y| of the oracle's exact value (and within one FP16 ulp
element by element). Small cases span several tiles and ragged tails; the
edge cases cover empty inputs, zero and constant rows, scale underflow and the
largest K.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_qoq_amd as qoq
from quantized_gemm_qoq_amd import workloads

from gpu_util import (DEV, assert_y_close, f16_dev, host, host_bits, quantize_all, to_dev)

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

G128, PC = qoq.MODE_G128, qoq.MODE_PER_CHANNEL
MODES = [G128, PC]


def _rand_bits(shape, seed, scale):
    return workloads.random_fp16(shape, seed, scale).numpy().view(np.uint16)


def _special_rows(x_bits):
    """Overwrite a few rows with edge cases (when there are enough rows)."""
    x = x_bits.copy()
    M, K = x.shape
    if M > 1:
        x[1] = 0  # all zero
    if M > 2:
        x[2] = np.float16(0.75).view(np.uint16)  # constant
    if M > 3:
        x[3] = 0
        x[3, K // 3] = np.float16(-3.0).view(np.uint16)  # single element
    if M > 4:
        x[4] = 0
        x[4, 5] = 0x0003  # subnormal maximum: the FP16 scale underflows to 0
    if M > 5:
        x[5] = (x[5].view(np.float16) * np.float16(0.001)).view(np.uint16)  # small values
    return x


# ------------------------------------------------------------ activations --
# K covers each register-resident row size (up to 4096, 8192, 16384 and 32768
# inputs per row, ragged within them), the first size above them, and the
# largest K; from 1024 rows (one wave per row) each of its register sizes (up
# to 2048, 4096, 8192 and 16384 inputs), ragged rows, and the first K above.
@pytest.mark.parametrize("M,K", [(1, 128), (7, 384), (64, 4096), (300, 1152), (5, 8192),
                                 (4, 14336), (3, 24576), (2, 32768 + 128), (3, 132096),
                                 (1030, 1152), (1024, 4096), (1040, 8192 - 128), (1025, 16384),
                                 (1024, 16384 + 128)])
def test_quantize_act(M, K):
    xb = _special_rows(_rand_bits((M, K), 10 + M, 1.0))
    print(f"quantize_act M={M} K={K}", flush=True)
    want_xq, want_sx, want_rs = oracle.quantize_act(xb)
    xq, s_x, rowsum = qoq.qoq_quantize_act(f16_dev(xb))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(xq), oracle.pack_act(want_xq))
    np.testing.assert_array_equal(host_bits(s_x), want_sx)
    np.testing.assert_array_equal(host(rowsum), want_rs)


def test_quantize_act_without_rowsum_and_empty():
    xb = _rand_bits((5, 256), 3, 2.0)
    xq, s_x, rs = qoq.qoq_quantize_act(f16_dev(xb), want_rowsum=False)
    torch.cuda.synchronize()
    assert rs is None
    np.testing.assert_array_equal(host(xq), oracle.pack_act(oracle.quantize_act(xb)[0]))
    e = torch.empty((0, 256), dtype=torch.float16, device=DEV)
    xq, s_x, rs = qoq.qoq_quantize_act(e)
    assert xq.numel() == 0


# ---------------------------------------------------------------- weights --
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("N,K", [(16, 128), (48, 640), (256, 4096), (32, 132096)])
def test_quantize_weights(mode, N, K):
    wb = _special_rows(_rand_bits((N, K), 20 + N, 0.02))
    if N > 8:
        wb[8, 7] = np.float16(0.9).view(np.uint16)  # an outlier
    print(f"quantize_weights mode={mode} N={N} K={K}", flush=True)
    want = oracle.quantize_weights(mode, wb)
    q, s_c, s_g, z = qoq.qoq_quantize_weights(mode, f16_dev(wb))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(q), want["q"])
    np.testing.assert_array_equal(host_bits(s_c), want["s_c"])
    np.testing.assert_array_equal(host(z), want["z"])
    if mode == G128:
        np.testing.assert_array_equal(host(s_g), want["s_g"])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("N,K", [(16, 128), (48, 640), (96, 2176)])
def test_pack_and_unpack(mode, N, K):
    wb = _rand_bits((N, K), 30 + K, 0.02)
    want = oracle.quantize_weights(mode, wb)
    want_blob = oracle.pack(mode, want["q"], want["s_g"], want["z"])
    print(f"pack mode={mode} N={N} K={K}", flush=True)
    sg = None if want["s_g"] is None else to_dev(want["s_g"])
    blob = qoq.qoq_pack_weights(mode, to_dev(want["q"]), sg, to_dev(want["z"]))
    q2, sg2, z2 = qoq.qoq_unpack_weights(mode, blob, N, K)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(blob), want_blob)
    np.testing.assert_array_equal(host(q2), want["q"])
    np.testing.assert_array_equal(host(z2), want["z"])
    if mode == G128:
        np.testing.assert_array_equal(host(sg2), want["s_g"])


# ------------------------------------------------------------------- GEMM --
GEMM_SHAPES = [
    (1, 16, 128), (8, 256, 512), (17, 48, 384), (64, 96, 1152), (100, 160, 256),
    (129, 32, 640), (257, 80, 128), (512, 512, 1024), (520, 272, 640), (3, 16, 132096),
    # streaming-kernel ring: main loop plus a leftover group, for 1, 2 and 4 row blocks
    (9, 32, 128 * 21), (30, 48, 128 * 67), (48, 64, 128 * 70),
    # streaming kernel with 64-row workgroups over bands of four channel
    # tiles (between 3/4 and one round): fewer groups than waves and a ragged
    # row block; a ragged last band and 9 groups over 8 waves; a last row
    # block of one row
    (72, 6144, 640), (256, 4080, 128 * 9), (129, 4096, 128 * 3),
    # split K over 4 uneven group ranges (13 groups) on 128 x 128 blocks,
    # ragged rows and channels
    (200, 272, 128 * 13),
    # 128 x 128 blocks, two workgroups per CU, K split 8 ways (33 groups)
    (130, 1040, 128 * 33),
    # LDS-pipelined kernel, 128-row blocks: group counts 0, 1 and 2 past a
    # multiple of its three-buffer loop, ragged rows and channels
    (600, 528, 128 * 9), (700, 400, 128 * 10), (200, 16400, 128 * 3),
    # ... one and two groups, one and three channel tiles
    (520, 16, 128), (1024, 48, 256),
    # the wide kernel: too many blocks for one round, ragged rows and channels
    (1024, 8208, 128 * 13), (640, 16400, 128 * 5),
    # ... with a ragged last block of rows, of channels, at 2 to 3 rounds of
    # blocks
    (520, 32784, 128 * 3), (1100, 16384, 128 * 2),
    # the large-block persistent kernel: one round of 256 x 256 blocks with
    # ragged rows and channels; two rounds (each workgroup crosses a block
    # boundary every 4 groups); 12 groups
    (4000, 4000, 128 * 8), (4000, 8000, 128 * 4), (2048, 8192, 128 * 12),
    # ... with a partial last round (384 blocks: half the workgroups take two)
    (1000, 24560, 128 * 4),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_against_oracle(mode, M, N, K):
    xb = _special_rows(_rand_bits((M, K), 40 + M + K, 1.0))
    # keep |Y| mostly inside the FP16 range at the largest K
    wb = _special_rows(_rand_bits((N, K), 50 + N + K, 0.02 if K < 65536 else 0.002))
    xq, s_x, rowsum, wq, blob = quantize_all(mode, xb, wb)
    acc_want = oracle.gemm(mode, xq, wq["q"], wq["s_g"], wq["z"])
    y_want = oracle.epilogue(acc_want, s_x, wq["s_c"])
    print(f"gemm mode={mode} M={M} N={N} K={K}", flush=True)
    d_xq, d_sx, d_rs = to_dev(oracle.pack_act(xq)), to_dev(s_x, torch.float16), to_dev(rowsum)
    d_blob, d_sc = to_dev(blob), to_dev(wq["s_c"], torch.float16)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y_acc = qoq.qoq_w4a8_gemm(mode, d_xq, d_sx, d_rs, d_blob, d_sc, N, acc_out=acc)
    y = qoq.qoq_w4a8_gemm(mode, d_xq, d_sx, d_rs if mode == PC else None, d_blob, d_sc, N)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(acc), acc_want)
    assert_y_close(host_bits(y), y_want, "fast path")
    np.testing.assert_array_equal(host_bits(y_acc), host_bits(y))


@pytest.mark.parametrize("mode", MODES)
def test_full_path_on_gpu(mode):
    """Every step on the GPU (quantize, pack, quantize_act, GEMM) against the
    oracle's end-to-end result."""
    M, N, K = 33, 272, 768
    xb = _special_rows(_rand_bits((M, K), 61, 1.0))
    wb = _rand_bits((N, K), 62, 0.02)
    res = oracle.forward(mode, xb, wb)
    pw = qoq.PackedWeight(mode, f16_dev(wb))
    y = pw.forward(f16_dev(xb))
    torch.cuda.synchronize()
    assert_y_close(host_bits(y), res["y"], "end to end")


def test_gemm_empty_and_zero_inputs():
    K, N = 256, 32
    wb = _rand_bits((N, K), 70, 0.02)
    for mode in MODES:
        pw = qoq.PackedWeight(mode, f16_dev(wb))
        y = pw.forward(torch.empty((0, K), dtype=torch.float16, device=DEV))
        assert y.shape == (0, N)
        y = pw.forward(torch.zeros((5, K), dtype=torch.float16, device=DEV))
        torch.cuda.synchronize()
        assert torch.all(y == 0)


def test_gemm_is_deterministic():
    M, N, K = 200, 256, 1024
    xb = _rand_bits((M, K), 80, 1.0)
    wb = _rand_bits((N, K), 81, 0.02)
    pw = qoq.PackedWeight(G128, f16_dev(wb))
    x = f16_dev(xb)
    y0 = pw.forward(x).clone()
    for _ in range(3):
        assert torch.equal(pw.forward(x), y0)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,K", [(64, 6144, 4096), (16, 8192, 8192), (40, 1040, 2048), (5, 400, 640),
                                   (256, 512, 2048), (100, 1040, 1152), (300, 2048, 640)])
def test_workspace_argument_leaves_results_unchanged(mode, M, N, K):
    """With a workspace of qoq_gemm_workspace_bytes() bytes the plan may split
    K (M > 64 with few output blocks); the accumulators and outputs must equal
    those of the unsplit plan (no workspace) bit for bit, twice in a row with
    the workspace reused (first filled with junk), and the packed activations
    must match the oracle's layout."""
    xb = _rand_bits((M, K), 90 + M, 1.0)
    wb = _rand_bits((N, K), 91 + N, 0.02)
    pw = qoq.PackedWeight(mode, f16_dev(wb))
    xq, s_x, rs = qoq.qoq_quantize_act(f16_dev(xb))
    need = qoq.qoq_gemm_workspace_bytes(mode, M, N, K)
    print(f"workspace mode={mode} M={M} N={N} K={K} ws={need}", flush=True)
    assert need >= 0
    a0 = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y0 = qoq.qoq_w4a8_gemm(mode, xq, s_x, rs, pw.blob, pw.s_c, N, acc_out=a0, workspace=None)
    ws = torch.full((max(16, need),), 0x5A, dtype=torch.uint8, device=DEV)
    for _ in range(2):
        a1 = torch.empty((M, N), dtype=torch.int32, device=DEV)
        y1 = qoq.qoq_w4a8_gemm(mode, xq, s_x, rs, pw.blob, pw.s_c, N, acc_out=a1, workspace=ws)
        y2 = qoq.qoq_w4a8_gemm(mode, xq, s_x, rs, pw.blob, pw.s_c, N, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a0, a1)
        assert torch.equal(y0, y1) and torch.equal(y0, y2)
    if M * N * K <= 4e8:
        xq_rm = oracle.quantize_act(xb)[0]
        np.testing.assert_array_equal(host(xq), oracle.pack_act(xq_rm))


def _oracle_w(mode, wb):
    wq = oracle.quantize_weights(mode, wb)
    return wq["q"], wq["s_g"], wq["z"]


def test_scales_exhaustive_over_fp16_row_max():
    """Every positive finite FP16 value as the largest magnitude of a row: the
    per-token scale max/127 and the per-channel scale max/119 (and the codes of
    the row's largest element) match the oracle bit for bit. This pins the
    GPU's division by a constant and the FP16 rounding of the scale."""
    vals = np.arange(1, 0x7C00, dtype=np.uint16)  # all positive finite FP16
    R = vals.size
    x = np.zeros((R, 128), np.uint16)
    x[:, 0] = vals
    x[:, 1] = vals | 0x8000  # the negative of the maximum
    x[:, 2] = np.maximum(vals, 1) - 1  # just below the maximum
    print(f"exhaustive scales over {R} rows", flush=True)
    want_xq, want_sx, want_rs = oracle.quantize_act(x)
    xq, s_x, rs = qoq.qoq_quantize_act(f16_dev(x))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(s_x), want_sx)
    np.testing.assert_array_equal(host(xq), oracle.pack_act(want_xq))
    np.testing.assert_array_equal(host(rs), want_rs)
    rows = (R + 15) // 16 * 16
    w = np.zeros((rows, 128), np.uint16)
    w[:R] = x
    for mode in MODES:
        want = oracle.quantize_weights(mode, w)
        q, s_c, s_g, z = qoq.qoq_quantize_weights(mode, f16_dev(w))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(s_c), want["s_c"])
        np.testing.assert_array_equal(host(q), want["q"])
        np.testing.assert_array_equal(host(z), want["z"])
        if mode == G128:
            np.testing.assert_array_equal(host(s_g), want["s_g"])


def _decode_channel_codes(tile_band, n, G):
    """Codes q[n, 0:128*G] of channel n from the bytes of its tile band
    (all G tiles of channels 16*(n//16) .. +15), walking the packed layout of
    include/qoq.h backwards: lane 16*j + c, byte 16*lane + 4*d + e holds kappa
    8*d + e (low nibble) and 8*d + 4 + e (high nibble), kappa = 16*s + i, input
    k = 128*g + 64*s + 16*j + i."""
    c = n % 16
    tiles = tile_band.reshape(G, 64, 16)
    q = np.zeros(128 * G, np.int64)
    for j in range(4):
        lane = tiles[:, 16 * j + c, :].astype(np.int64)  # [G, 16]
        for b in range(16):
            d, e = divmod(b, 4)
            for half in range(2):
                kappa = 8 * d + 4 * half + e
                s, i = divmod(kappa, 16)
                k = 128 * np.arange(G) + 64 * s + 16 * j + i
                q[k] = (lane[:, b] >> (4 * half)) & 15
    return q


def test_gemm_blob_of_2gib_takes_the_64bit_path():
    """A weight blob of 2 GiB or more does not fit the buffer-load kernels'
    31-bit offsets; the plan then falls back to the reference kernel (M <= 64),
    which addresses with 64-bit pointers. Random codes (any nibble is a valid
    per-channel code) and random zeros; accumulators and outputs are checked at
    sampled channels, including the last one, against an independent decode of
    the blob on the host."""
    M, N, K = 2, 32768, 131072
    G = K // 128
    code_bytes = N * K // 2
    assert code_bytes >= 1 << 31
    print(f"2 GiB blob: M={M} N={N} K={K}", flush=True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    blob = torch.randint(0, 256, (qoq.qoq_packed_bytes(PC, N, K),), dtype=torch.uint8,
                         device=DEV, generator=gen)
    blob[code_bytes:] = torch.randint(0, 16, (N,), dtype=torch.uint8, device=DEV, generator=gen)
    s_c = to_dev(workloads.random_fp16((N,), 8, 1e-3).numpy().view(np.uint16), torch.float16)
    xb = _rand_bits((M, K), 9, 1.0)
    xq, s_x, rowsum = qoq.qoq_quantize_act(f16_dev(xb))
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y = qoq.qoq_w4a8_gemm(PC, xq, s_x, rowsum, blob, s_c, N, acc_out=acc)
    torch.cuda.synchronize()
    oxq, osx, _ = oracle.quantize_act(xb)
    z_all = host(blob[code_bytes:])
    sc_bits = host_bits(s_c)
    acc_h, y_h = host(acc), host_bits(y)
    for n in (0, 1, 15, 16, 12345, N - 17, N - 1):
        t = n // 16
        band = host(blob[t * G * 1024:(t + 1) * G * 1024])
        q = _decode_channel_codes(band, n, G)
        want = oxq.astype(np.int64) @ (q - int(z_all[n]))
        np.testing.assert_array_equal(acc_h[:, n], want)
        y_want = oracle.epilogue(want.astype(np.int32)[:, None], osx,
                                 np.array([sc_bits[n]], np.uint16))[:, 0]
        assert_y_close(y_h[:, n][:, None], y_want[:, None], f"channel {n}")
    del blob
    torch.cuda.empty_cache()
