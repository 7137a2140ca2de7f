"""Host-side checks of the GPU design, run on the CPU with numpy.

The GPU main loop unpacks four UINT4 codes per 32-bit word to INT8 with three
integer operations (the pages' "multiply by the integer scale, then subtract
the precomputed zero-point compensation", done four lanes at a time inside one
register):

    P  = word & 0x0F0F0F0F            (or (word >> 4) & 0x0F0F0F0F)
    T  = v_pk_mad_u16(P, s_g * 0x00010001, C * 0x00010001)
         with C = ((128 - z * s_g) * 257) mod 2^16
    W8 = T ^ 0x80808080

Each byte of T is (q - z) * s_g + 128, which lies in [0, 255] exactly when the
unpacked value lies in INT8; the XOR turns the biased byte into two's
complement. The protective range [-119, 119] is what guarantees that case.

The second test emulates, in numpy, how the GEMM kernel pairs activation bytes
with unpacked weight bytes on the matrix cores for the packed layout written
out in include/qoq.h, and checks the result against the oracle's definition
of the accumulator.
"""
import numpy as np
import pytest

import oracle
from quantized_gemm_qoq_amd import workloads

G128 = oracle.MODE_G128
PC = oracle.MODE_PER_CHANNEL


def pk_mad_u16(a, b, c):
    """v_pk_mad_u16: per 16-bit half, a*b + c modulo 2^16 (no clamp)."""
    a = a.astype(np.uint64)
    b = b.astype(np.uint64)
    c = c.astype(np.uint64)
    lo = ((a & 0xFFFF) * (b & 0xFFFF) + (c & 0xFFFF)) & 0xFFFF
    hi = (((a >> 16) & 0xFFFF) * ((b >> 16) & 0xFFFF) + ((c >> 16) & 0xFFFF)) & 0xFFFF
    return (lo | (hi << 16)).astype(np.uint32)


def swar_unpack(codes_word, s_g, z):
    """codes_word holds four codes, one per byte (0x0q0q0q0q)."""
    s_g = np.asarray(s_g, np.uint32)
    z = np.asarray(z, np.uint32)
    mul = s_g * np.uint32(0x00010001)
    c16 = ((128 - (z.astype(np.int64) * s_g.astype(np.int64))) * 257) & 0xFFFF
    add = (c16.astype(np.uint32) * np.uint32(0x00010001)).astype(np.uint32)
    return pk_mad_u16(codes_word, mul, add) ^ np.uint32(0x80808080)


def test_swar_unpack_exhaustive():
    quads = np.arange(65536, dtype=np.uint32)
    q = np.stack([(quads >> (4 * i)) & 15 for i in range(4)])  # [4, 65536]
    word = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24)
    total_valid = 0
    for s_g in range(1, 17):
        for z in range(16):
            r = swar_unpack(word, s_g, z)
            got = np.stack([((r >> (8 * i)) & 0xFF).astype(np.uint8).view(np.int8) for i in range(4)])
            want = (q.astype(np.int64) - z) * s_g
            valid = np.all((want >= -128) & (want <= 127), axis=0)
            total_valid += int(valid.sum())
            np.testing.assert_array_equal(got[:, valid].astype(np.int64), want[:, valid])
            # Every quadruple the quantizer can emit is valid: |(q - z) s_g| <= 121.
            emit = np.all(np.abs(want) <= 121, axis=0)
            assert np.all(valid[emit])
    assert total_valid > 13_000_000


def _operand_bytes(words):
    """words [..., 4] uint32 -> [..., 16] int8 (little-endian bytes)."""
    return np.ascontiguousarray(words.astype(np.uint32)).view(np.uint8).view(np.int8)


def emulate_gemm(mode, xq, blob, rowsum, N, K):
    """Emulate the kernel's operand assembly over the packed blob and the
    packed activations: lane l of an MFMA 16x16x64 step holds row/column
    l % 16 and bytes 16*(l // 16) .. +15 of the 64-wide k slice, for both
    operands; the A operand of tile (g, u), k-step s is the 1 KB at
    (g * Mp/16 + u) * 2048 + 1024 * s of the packed activations."""
    M = xq.shape[0]
    apk = oracle.pack_act(xq)
    G = K // 128
    T = N // 16
    words = np.ascontiguousarray(blob[: N * K // 2]).view(np.uint32).reshape(T, G, 64, 4)
    params = blob[N * K // 2:]
    Mp = (M + 15) // 16 * 16
    xpad = np.zeros((Mp, K), np.int8)
    xpad[:M] = xq
    acc = np.zeros((Mp, N), np.int64)
    lanes = np.arange(64)
    c = lanes % 16
    j = lanes // 16
    for t in range(T):
        n = 16 * t + c  # channel of each lane
        for g in range(G):
            w = words[t, g]  # [64, 4]
            if mode == G128:
                # 16 parameter bytes per (tile, group), one per channel
                p = params[(t * G + g) * 16 + c].astype(np.uint32)
                s_g, z = (p >> 4) + 1, p & 15
            for s in range(2):
                P0, P1 = w[:, 2 * s], w[:, 2 * s + 1]
                ops = np.stack([P0 & 0x0F0F0F0F, (P0 >> 4) & 0x0F0F0F0F,
                                P1 & 0x0F0F0F0F, (P1 >> 4) & 0x0F0F0F0F], axis=1).astype(np.uint32)
                if mode == G128:
                    ops = swar_unpack(ops, s_g[:, None], z[:, None])
                b = _operand_bytes(ops).astype(np.int64)  # [64 lanes, 16]
                k0 = 128 * g + 64 * s
                for mb in range(Mp // 16):
                    off = (g * (Mp // 16) + mb) * 2048 + 1024 * s
                    a = apk[off:off + 1024].reshape(64, 16).astype(np.int64)
                    # the same operand read from the row-major values directly
                    rows = 16 * mb + c
                    a_rm = np.stack([xpad[rows[l], k0 + 16 * j[l]: k0 + 16 * j[l] + 16] for l in range(64)])
                    np.testing.assert_array_equal(a, a_rm)
                    # D[i][jj] = sum over lane groups jg and bytes of A[i + 16 jg] * B[jj + 16 jg]
                    d = np.zeros((16, 16), np.int64)
                    for jg in range(4):
                        d += a[16 * jg:16 * jg + 16] @ b[16 * jg:16 * jg + 16].T
                    acc[16 * mb:16 * mb + 16, 16 * t:16 * t + 16] += d
    acc = acc[:M]
    if mode == PC:
        acc -= np.outer(rowsum.astype(np.int64), params[:N].astype(np.int64))
    return acc


@pytest.mark.parametrize("mode", [G128, PC])
def test_mfma_operand_emulation_matches_oracle(mode):
    M, K, N = 21, 384, 48
    x = workloads.random_fp16((M, K), 41, 1.0).numpy().view(np.uint16)
    w = workloads.random_fp16((N, K), 42, 0.02).numpy().view(np.uint16)
    xq, s_x, rowsum = oracle.quantize_act(x)
    wq = oracle.quantize_weights(mode, w)
    blob = oracle.pack(mode, wq["q"], wq["s_g"], wq["z"])
    want = oracle.gemm(mode, xq, wq["q"], wq["s_g"], wq["z"])
    got = emulate_gemm(mode, xq, blob, rowsum, N, K)
    np.testing.assert_array_equal(got, want)


def test_pack_spec_round_trip_independent_decode():
    """Decode the blob by walking the layout in the opposite direction (tile,
    lane, byte, nibble -> n, k) and recover the codes and parameters."""
    N, K = 32, 640
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    G = K // 128
    s_g = rng.integers(1, 17, size=(N, G), dtype=np.uint8)
    z = rng.integers(0, 16, size=(N, G), dtype=np.uint8)
    blob = oracle.pack(G128, q, s_g, z)
    back = np.full((N, K), 255, np.uint8)
    for t in range(N // 16):
        for g in range(G):
            tile = blob[(t * G + g) * 1024:(t * G + g + 1) * 1024]
            for lane in range(64):
                c, j = lane % 16, lane // 16
                for byte in range(16):
                    d, e = divmod(byte, 4)
                    for half in range(2):
                        kappa = 8 * d + 4 * half + e
                        s, i = divmod(kappa, 16)
                        k = 128 * g + 64 * s + 16 * j + i
                        back[16 * t + c, k] = (tile[16 * lane + byte] >> (4 * half)) & 15
    np.testing.assert_array_equal(back, q)
    assert blob.size == N * K // 2 + N * G
    # parameters: [tile][group][16 channels]
    params = blob[N * K // 2:].reshape(N // 16, G, 16).transpose(0, 2, 1).reshape(N, G)
    np.testing.assert_array_equal((params >> 4) + 1, s_g)
    np.testing.assert_array_equal(params & 15, z)
