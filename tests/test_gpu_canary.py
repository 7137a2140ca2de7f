"""Guard canaries around every output of every entry point: each output buffer
is the middle of a larger allocation whose bytes before and after it hold a
sentinel, and after the call (and a synchronization) every sentinel byte must
be unchanged. The shapes are ragged in M (row tiles of 16 only partly used)
and in N, and they reach every GEMM plan: the streaming decode kernel, the
16-row-wave tiled kernel without a workspace, the LDS-pipelined kernel with
and without split K, and the wide kernel. The outputs themselves are checked
against the oracle elsewhere; here the point is that no kernel writes outside
the bytes its arguments give it (including the padded activation rows, the
split-K partial sums and the split-row tallies)."""
import numpy as np
import pytest
import torch

import quantized_gemm_qoq_amd as qoq
from quantized_gemm_qoq_amd import workloads

from gpu_util import DEV

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

GUARD = 4096  # sentinel bytes on each side
SENTINEL = 0xA5


class Guarded:
    """nbytes of device memory (viewed as dtype/shape) between two guard zones."""

    def __init__(self, nbytes, dtype=torch.uint8, shape=None):
        self.nbytes = int(nbytes)
        self.buf = torch.full((GUARD + self.nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device=DEV)
        mid = self.buf[GUARD:GUARD + self.nbytes]
        t = mid.view(dtype)
        self.t = t.view(shape) if shape is not None else t

    def check(self, what):
        torch.cuda.synchronize()
        lo = self.buf[:GUARD]
        hi = self.buf[GUARD + self.nbytes:]
        assert bool((lo == SENTINEL).all()), f"{what}: bytes before the buffer were written"
        assert bool((hi == SENTINEL).all()), f"{what}: bytes after the buffer were written"


def _f16(shape, seed, scale):
    return workloads.random_fp16(shape, seed, scale).to(DEV)


# (M, K, N) reaching: stream (M <= 64, and 64-row workgroups at 72 rows),
# tiled without workspace, LDS-pipelined split-K with workspace, LDS-pipelined
# unsplit, wide.
GEMM_CASES = [(1, 256, 48), (17, 384, 272), (33, 640, 16), (63, 256, 528), (72, 640, 6144),
              (65, 512, 272), (130, 1024, 144), (200, 1664, 272), (257, 256, 48),
              (600, 1152, 528), (640, 640, 16400)]


@pytest.mark.parametrize("M,K,N", GEMM_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("mode", ["g128", "per_channel", "w8a8"])
def test_gemm_and_act_quant_write_only_their_outputs(mode, M, K, N):
    w = _f16((N, K), 40 + N, 0.02)
    pw = qoq.PackedWeight(mode, w)
    x = _f16((M, K), 41 + M, 1.0)
    # activation quantization
    xq = Guarded(qoq.qoq_act_bytes(M, K), torch.int8)
    s_x = Guarded(2 * M, torch.float16)
    rowsum = Guarded(4 * M, torch.int32)
    qoq.qoq_quantize_act(x, xq.t, s_x.t, rowsum.t)
    for g, name in ((xq, "xq"), (s_x, "s_x"), (rowsum, "rowsum")):
        g.check(f"qoq_quantize_act {name}")
    # the GEMM, with and without accumulator output, with and without workspace
    if mode == qoq.W8A8:
        need = qoq.qoq_w8a8_gemm_workspace_bytes(M, N, K)
    else:
        need = qoq.qoq_gemm_workspace_bytes(mode, M, N, K)
    for use_ws in ((False, True) if need > 0 else (False,)):
        y = Guarded(2 * M * N, torch.float16, (M, N))
        acc = Guarded(4 * M * N, torch.int32, (M, N))
        ws = Guarded(need) if use_ws else None
        if mode == qoq.W8A8:
            qoq.qoq_w8a8_gemm(xq.t, s_x.t, pw.blob, pw.s_c, N, y=y.t, acc_out=acc.t,
                              workspace=ws.t if ws else None, K=K)
        else:
            rs = rowsum.t if mode == "per_channel" else None
            qoq.qoq_w4a8_gemm(mode, xq.t, s_x.t, rs, pw.blob, pw.s_c, N, y=y.t, acc_out=acc.t,
                              workspace=ws.t if ws else None, K=K)
        y.check(f"gemm y ws={use_ws}")
        acc.check(f"gemm acc_out ws={use_ws}")
        if ws:
            ws.check("gemm workspace")
        # the fast path (no accumulator output) writes the same outputs
        y2 = Guarded(2 * M * N, torch.float16, (M, N))
        if mode == qoq.W8A8:
            qoq.qoq_w8a8_gemm(xq.t, s_x.t, pw.blob, pw.s_c, N, y=y2.t,
                              workspace=ws.t if ws else None, K=K)
        else:
            qoq.qoq_w4a8_gemm(mode, xq.t, s_x.t, rs, pw.blob, pw.s_c, N, y=y2.t,
                              workspace=ws.t if ws else None, K=K)
        y2.check("gemm fast-path y")
        assert torch.equal(y.t, y2.t)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (272, 1152)])
@pytest.mark.parametrize("mode", ["g128", "per_channel"])
def test_weight_quantize_pack_unpack_write_only_their_outputs(mode, N, K):
    m = qoq.MODES[mode]
    w = _f16((N, K), 60 + N, 0.02)
    G = K // 128
    q = Guarded(N * K, torch.uint8, (N, K))
    s_c = Guarded(2 * N, torch.float16)
    zn = N * G if m == qoq.MODE_G128 else N
    s_g = Guarded(N * G, torch.uint8, (N, G)) if m == qoq.MODE_G128 else None
    z = Guarded(zn, torch.uint8, (N, G) if m == qoq.MODE_G128 else (N,))
    qoq.qoq_quantize_weights(m, w, q.t, s_c.t, s_g.t if s_g else None, z.t)
    for g, name in ((q, "q"), (s_c, "s_c"), (s_g, "s_g"), (z, "z")):
        if g is not None:
            g.check(f"qoq_quantize_weights {name}")
    blob = Guarded(qoq.qoq_packed_bytes(m, N, K))
    qoq.qoq_pack_weights(m, q.t, s_g.t if s_g else None, z.t, blob.t)
    blob.check("qoq_pack_weights blob")
    # unpack into guarded outputs through the C ABI directly
    lib = qoq.load_library()
    q2 = Guarded(N * K)
    sg2 = Guarded(N * G) if m == qoq.MODE_G128 else None
    z2 = Guarded(zn)
    st = lib.qoq_unpack_weights(m, qoq._ptr(blob.t), N, K, qoq._ptr(q2.t),
                                qoq._ptr(sg2.t) if sg2 else None, qoq._ptr(z2.t), qoq._stream(blob.t))
    assert st == 0
    for g, name in ((q2, "q"), (sg2, "s_g"), (z2, "z")):
        if g is not None:
            g.check(f"qoq_unpack_weights {name}")
    assert torch.equal(q2.t.view(N, K), q.t)


@pytest.mark.parametrize("M,I", [(1, 256), (17, 640), (16, 12288), (33, 14336)])
def test_producers_write_only_their_outputs(M, I):
    gu = _f16((M, 2 * I), 70 + M, 2.0)
    lib = qoq.load_library()
    for use_ws in (False, True):
        xq = Guarded(qoq.qoq_act_bytes(M, I), torch.int8)
        s_x = Guarded(2 * M, torch.float16)
        rs = Guarded(4 * M, torch.int32)
        h = Guarded(2 * M * I, torch.float16, (M, I))
        need = int(lib.qoq_silu_mul_workspace_bytes(M, I))
        ws = Guarded(need) if (use_ws and need > 0) else None
        qoq.qoq_silu_mul_quantize_act(gu, xq.t, s_x.t, rs.t, h=h.t, workspace=ws.t if ws else None)
        for g, name in ((xq, "xq"), (s_x, "s_x"), (rs, "rowsum"), (h, "h"), (ws, "workspace")):
            if g is not None:
                g.check(f"silu producer {name} ws={use_ws}")
    if I <= 32768:
        x = _f16((M, I), 71 + M, 1.0)
        gamma = _f16((I,), 72, 0.5).abs() + 0.5
        xq = Guarded(qoq.qoq_act_bytes(M, I), torch.int8)
        s_x = Guarded(2 * M, torch.float16)
        rs = Guarded(4 * M, torch.int32)
        yn = Guarded(2 * M * I, torch.float16, (M, I))
        qoq.qoq_rmsnorm_quantize_act(x, gamma, 1e-5, xq.t, s_x.t, rs.t, y=yn.t)
        for g, name in ((xq, "xq"), (s_x, "s_x"), (rs, "rowsum"), (yn, "y")):
            g.check(f"rmsnorm producer {name}")


@pytest.mark.parametrize("M,K,N", [(1, 256, 48), (33, 640, 272), (130, 1024, 144), (600, 384, 528)])
def test_w4a16_writes_only_its_outputs(M, K, N):
    pw = qoq.PackedWeight("g128", _f16((N, K), 80 + N, 0.02))
    x = _f16((M, K), 81 + M, 1.0)
    y = Guarded(2 * M * N, torch.float16, (M, N))
    acc = Guarded(4 * M * N, torch.float32, (M, N))
    qoq.qoq_w4a16_gemm("g128", x, pw.blob, pw.s_c, N, y=y.t, acc_out=acc.t)
    y.check("w4a16 y")
    acc.check("w4a16 acc_out")


def test_kv4_entry_points_write_only_their_outputs():
    B, H, Hq, T, Tcap = 3, 4, 16, 50, 64
    d = qoq.HEAD_DIM
    k = _f16((B, T, H, d), 90, 1.0)
    v = _f16((B, T, H, d), 91, 1.0)
    lam = Guarded(2 * H * d, torch.float16, (H, d))
    lib = qoq.load_library()
    st = lib.qoq_kv4_smooth_scales(qoq._ptr(k[0]), T, H, d, qoq._ptr(lam.t), qoq._stream(k))
    assert st == 0
    lam.check("smooth scales")
    kq = Guarded(B * H * Tcap * 64)
    vq = Guarded(B * H * Tcap * 64)
    ks, vs = Guarded(2 * B * H * Tcap), Guarded(2 * B * H * Tcap)
    kz, vz = Guarded(B * H * Tcap), Guarded(B * H * Tcap)
    st = lib.qoq_kv4_append(qoq._ptr(k), qoq._ptr(v), qoq._ptr(lam.t), B, T, H, d, Tcap, 0,
                            qoq._ptr(kq.t), qoq._ptr(ks.t), qoq._ptr(kz.t), qoq._ptr(vq.t),
                            qoq._ptr(vs.t), qoq._ptr(vz.t), qoq._stream(k))
    assert st == 0
    for g, name in ((kq, "kq"), (vq, "vq"), (ks, "ks"), (vs, "vs"), (kz, "kz"), (vz, "vz")):
        g.check(f"kv4 append {name}")
    q = _f16((B, Hq, d), 92, 1.0)
    lens = torch.tensor([50, 17, 1], dtype=torch.int32, device=DEV)
    o = Guarded(2 * B * Hq * d, torch.float16, (B, Hq, d))
    need = int(lib.qoq_kv4_attention_workspace_bytes(B, Hq, H, d, Tcap))
    ws = Guarded(max(need, 16))
    st = lib.qoq_kv4_decode_attention(qoq._ptr(q), qoq._ptr(lam.t), qoq._ptr(kq.t), qoq._ptr(ks.t),
                                      qoq._ptr(kz.t), qoq._ptr(vq.t), qoq._ptr(vs.t), qoq._ptr(vz.t),
                                      qoq._ptr(lens), B, Hq, H, d, Tcap, qoq._ptr(o.t), qoq._ptr(ws.t),
                                      ws.nbytes, qoq._stream(q))
    assert st == 0
    o.check("kv4 attention o")
    ws.check("kv4 attention workspace")
