"""Host-only checks of the C ABI: the library loads, exports every entry point
that include/qoq.h declares, and rejects invalid arguments before launching
anything (no call here reaches a kernel, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

import quantized_gemm_qoq_amd as qoq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qoq.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_MODE, ERR_HIP, ERR_WORKSPACE, ERR_HEADER = range(8)
A = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every call below fails validation
U = ctypes.c_void_p(0x10004)  # misaligned
NUL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qoq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return qoq.load_library()


def test_exports_every_declared_symbol(lib):
    decl = declared_functions()
    assert decl == sorted(qoq.EXPORTED)
    for name in decl:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    hdr = open(HEADER).read()
    ver = int(re.search(r"#define QOQ_ABI_VERSION (\d+)", hdr).group(1))
    assert lib.qoq_abi_version() == ver == qoq.qoq_abi_version()
    for s in range(8):
        assert lib.qoq_status_str(s) and lib.qoq_status_str(s) != b"unknown status"
    assert lib.qoq_status_str(99) == b"unknown status"


def test_packed_bytes(lib):
    assert lib.qoq_packed_bytes(0, 16, 128) == 16 * 64 + 16
    assert lib.qoq_packed_bytes(1, 16, 128) == 16 * 64 + 16
    assert lib.qoq_packed_bytes(0, 6144, 4096) == 6144 * 2048 + 6144 * 32
    assert lib.qoq_packed_bytes(0, 32, 128 * 17) == 32 * 64 * 17 + 32 * 17
    assert lib.qoq_packed_bytes(0, 15, 128) == -1
    assert lib.qoq_packed_bytes(0, 16, 129) == -1
    assert lib.qoq_packed_bytes(0, 16, 132096 + 128) == -1
    assert lib.qoq_packed_bytes(2, 16, 128) == -1


def test_act_bytes(lib):
    assert lib.qoq_act_bytes(1, 128) == 16 * 128
    assert lib.qoq_act_bytes(16, 256) == 16 * 256
    assert lib.qoq_act_bytes(17, 256) == 32 * 256
    assert lib.qoq_act_bytes(0, 128) == 0
    assert lib.qoq_act_bytes(4, 100) == -1


def test_quantize_act_validation(lib):
    f = lib.qoq_quantize_act
    assert f(A, 0, 128, A, A, A, NUL) == OK  # empty: nothing launched
    assert f(NUL, 0, 128, NUL, NUL, NUL, NUL) == OK
    assert f(A, -1, 128, A, A, A, NUL) == ERR_SHAPE
    assert f(A, 4, 100, A, A, A, NUL) == ERR_SHAPE
    assert f(A, 4, 0, A, A, A, NUL) == ERR_SHAPE
    assert f(A, 4, 132096 + 128, A, A, A, NUL) == ERR_SHAPE
    assert f(NUL, 4, 128, A, A, A, NUL) == ERR_NULL
    assert f(A, 4, 128, NUL, A, A, NUL) == ERR_NULL
    assert f(A, 4, 128, A, NUL, A, NUL) == ERR_NULL
    assert f(U, 4, 128, A, A, A, NUL) == ERR_ALIGN
    assert f(A, 4, 128, A, A, U, NUL) == ERR_ALIGN


def test_quantize_weights_validation(lib):
    f = lib.qoq_quantize_weights
    assert f(2, A, 16, 128, A, A, A, A, NUL) == ERR_MODE
    assert f(0, A, 0, 128, NUL, NUL, NUL, NUL, NUL) == OK
    assert f(0, A, 15, 128, A, A, A, A, NUL) == ERR_SHAPE
    assert f(0, A, 16, 64, A, A, A, A, NUL) == ERR_SHAPE
    assert f(0, A, 16, 128, A, A, NUL, A, NUL) == ERR_NULL  # g128 needs s_g
    assert f(1, A, 16, 128, A, A, NUL, NUL, NUL) == ERR_NULL  # z always needed
    assert f(0, U, 16, 128, A, A, A, A, NUL) == ERR_ALIGN


def test_pack_unpack_validation(lib):
    p = lib.qoq_pack_weights
    u = lib.qoq_unpack_weights
    assert p(3, A, A, A, 16, 128, A, NUL) == ERR_MODE
    assert p(0, A, A, A, 0, 128, A, NUL) == ERR_SHAPE  # a blob needs at least one tile
    assert p(0, A, A, A, 24, 128, A, NUL) == ERR_SHAPE
    assert p(0, A, NUL, A, 16, 128, A, NUL) == ERR_NULL
    assert p(0, A, A, A, 16, 128, NUL, NUL) == ERR_NULL
    assert p(0, A, A, A, 16, 128, U, NUL) == ERR_ALIGN
    assert u(0, A, 16, 130, A, A, A, NUL) == ERR_SHAPE
    assert u(1, A, 16, 128, NUL, NUL, A, NUL) == ERR_NULL
    assert u(1, U, 16, 128, A, NUL, A, NUL) == ERR_ALIGN


def test_gemm_validation(lib):
    f = lib.qoq_w4a8_gemm
    def args(mode=0, xq=A, sx=A, rs=A, blob=A, sc=A, M=8, N=16, K=128, y=A, acc=NUL, ws=NUL,
             wsb=0):
        return f(mode, xq, sx, rs, blob, sc, M, N, K, y, acc, ws, wsb, NUL)
    assert args(mode=5) == ERR_MODE
    assert args(M=0) == OK
    assert args(N=0) == OK
    assert args(M=-2) == ERR_SHAPE
    assert args(N=8) == ERR_SHAPE
    assert args(K=256 + 64) == ERR_SHAPE
    assert args(K=132096 + 128) == ERR_SHAPE
    assert args(xq=NUL) == ERR_NULL
    assert args(y=NUL) == ERR_NULL
    assert args(mode=1, rs=NUL) == ERR_NULL  # per-channel needs the row sums
    assert args(blob=U) == ERR_ALIGN
    assert args(acc=U) == ERR_ALIGN
    assert args(ws=U, wsb=1 << 20) == ERR_ALIGN
    assert lib.qoq_gemm_workspace_bytes(0, 64, 6144, 4096) == 0  # decode plans need none
    need = lib.qoq_gemm_workspace_bytes(0, 256, 512, 2048)  # few blocks: split K
    assert need > 0 and need % (256 * 512 * 4) == 0
    assert args(M=256, N=512, K=2048, ws=A, wsb=need - 1) == ERR_WORKSPACE


def test_workspace_bytes(lib):
    f = lib.qoq_gemm_workspace_bytes
    assert f(2, 8, 16, 128) == -1
    assert f(0, 8, 15, 128) == -1
    assert f(0, 0, 16, 128) == 0
    assert f(0, 8, 16, 128) >= 0
    assert f(0, 64, 6144, 4096) % 16 == 0


def test_middle_m_split_plans(lib):
    """The K splits the plan picks for the middle-M benchmark layers, seen
    through the workspace they need (S * M * N INT32 partial sums): none where
    64-row streaming workgroups make 3/4 to one round (4-bit weights,
    M <= 256, K <= 16384); else 128 x 128 blocks of two workgroups per CU
    split in the smallest power of two that fills a round (4-bit weights,
    M < 512, K <= 16384), else 128 x 256 blocks split up to 8 ways."""
    f, w8 = lib.qoq_gemm_workspace_bytes, lib.qoq_w8a8_gemm_workspace_bytes
    part = lambda S, M, N: S * M * N * 4
    for mode in (0, 1):
        assert f(mode, 128, 8192, 8192) == 0                       # Qwen1.5-72B o_proj: 256 streams
        assert f(mode, 128, 4096, 8192) == part(8, 128, 4096)      # 128 streams: 32 blocks, 8 splits
        assert f(mode, 128, 24576, 8192) == part(2, 128, 24576)    # qkv: 192 blocks
        assert f(mode, 128, 49152, 8192) == 0                      # gate_up: 384 blocks, no split
        assert f(mode, 128, 8192, 24576) == part(8, 128, 8192)     # down, K > 16384: 32 wide blocks
        assert f(mode, 256, 4096, 14336) == 0                      # Llama-3-8B down: 256 streams
        assert f(mode, 256, 4096, 24576) == part(8, 256, 4096)     # K > 16384: 32 wide blocks, 8 splits
        assert f(mode, 256, 28672, 4096) == 0                      # Llama-3-8B gate_up: 448 blocks
    for mode in (0, 1):  # the GPU parity shapes of the 64-row streaming plan need no workspace
        assert f(mode, 72, 6144, 640) == f(mode, 256, 4080, 128 * 9) == f(mode, 129, 4096, 384) == 0
    assert w8(128, 8192, 8192) == part(8, 128, 8192)               # INT8 weights: 128 x 256 blocks
    assert f(0, 130, 1040, 128 * 33) == part(8, 130, 1040)         # 18 blocks: 8 splits of 33 groups
    assert f(0, 200, 272, 128 * 13) == part(4, 200, 272)           # 13 groups: at most 6 splits -> 4


def test_w8a8_validation(lib):
    assert lib.qoq_w8a8_packed_bytes(16, 128) == 16 * 128
    assert lib.qoq_w8a8_packed_bytes(15, 128) == -1
    assert lib.qoq_w8a8_packed_bytes(16, 100) == -1
    q = lib.qoq_w8a8_quantize_weights
    assert q(A, 0, 128, NUL, NUL, NUL) == OK
    assert q(A, 24, 128, A, A, NUL) == ERR_SHAPE
    assert q(A, 16, 128, NUL, A, NUL) == ERR_NULL
    assert q(U, 16, 128, A, A, NUL) == ERR_ALIGN
    p = lib.qoq_w8a8_pack_weights
    assert p(A, 0, 128, A, NUL) == ERR_SHAPE
    assert p(A, 16, 128, NUL, NUL) == ERR_NULL
    assert p(A, 16, 128, U, NUL) == ERR_ALIGN
    f = lib.qoq_w8a8_gemm
    def args(xq=A, sx=A, blob=A, sc=A, M=8, N=16, K=128, y=A, acc=NUL, ws=NUL, wsb=0):
        return f(xq, sx, blob, sc, M, N, K, y, acc, ws, wsb, NUL)
    assert args(M=0) == OK
    assert args(N=8) == ERR_SHAPE
    assert args(K=200) == ERR_SHAPE
    assert args(blob=NUL) == ERR_NULL
    assert args(y=U) == ERR_ALIGN
    w = lib.qoq_w8a8_gemm_workspace_bytes
    assert w(64, 6144, 4096) == 0
    need = w(256, 512, 2048)
    assert need > 0 and need % (256 * 512 * 4) == 0
    assert args(M=256, N=512, K=2048, ws=A, wsb=need - 1) == ERR_WORKSPACE
    assert w(8, 15, 128) == -1


def test_w4a16_validation(lib):
    f = lib.qoq_w4a16_gemm
    def args(mode=0, x=A, blob=A, sc=A, M=8, N=16, K=128, y=A, acc=NUL):
        return f(mode, x, blob, sc, M, N, K, y, acc, NUL)
    assert args(mode=3) == ERR_MODE
    assert args(M=0) == OK
    assert args(M=-1) == ERR_SHAPE
    assert args(N=24 + 1) == ERR_SHAPE
    assert args(K=384 + 64) == ERR_SHAPE
    assert args(x=NUL) == ERR_NULL
    assert args(sc=NUL) == ERR_NULL
    assert args(x=U) == ERR_ALIGN
    assert args(acc=U) == ERR_ALIGN


def test_silu_mul_quantize_validation(lib):
    f = lib.qoq_silu_mul_quantize_act
    assert f(A, 0, 128, A, A, A, NUL, NUL) == OK
    assert f(A, -1, 128, A, A, A, NUL, NUL) == ERR_SHAPE
    assert f(A, 4, 100, A, A, A, NUL, NUL) == ERR_SHAPE
    assert f(NUL, 4, 128, A, A, A, NUL, NUL) == ERR_NULL
    assert f(A, 4, 128, A, NUL, A, NUL, NUL) == ERR_NULL
    assert f(U, 4, 128, A, A, A, NUL, NUL) == ERR_ALIGN
    assert f(A, 4, 128, A, A, A, U, NUL) == ERR_ALIGN


def test_silu_mul_split_workspace(lib):
    w = lib.qoq_silu_mul_workspace_bytes
    # 24 shares of 1024 inputs per row: their maxima, then a 256-byte tally line per row
    assert w(16, 24576) == 16 * 24 * 4 + 16 * 256
    assert w(32, 14336) == 32 * 14 * 4 + 32 * 256
    assert w(64, 14336) == 0                # enough rows for the one-pass kernel
    assert w(16, 11008) == 0                # rows short enough for it
    assert w(16, 12288) == 16 * 12 * 4 + 16 * 256
    assert w(32, 12288) > 0 and w(33, 24576) == 0  # at most 32 rows (two row tiles) split
    assert w(512, 14336) == 0               # enough rows: one pass
    assert w(16, 512) == 0                  # rows too short to share
    assert w(16, 100) == -1
    f = lib.qoq_silu_mul_quantize_act_ws
    assert f(A, 16, 24576, A, A, A, NUL, A, 5631, NUL) == ERR_WORKSPACE  # workspace too small
    assert f(A, 16, 24576, A, A, A, NUL, U, 5632, NUL) == ERR_ALIGN
    assert f(A, 0, 24576, A, A, A, NUL, NUL, 0, NUL) == OK
    assert f(NUL, 16, 24576, A, A, A, NUL, A, 5632, NUL) == ERR_NULL


def test_rmsnorm_quantize_validation(lib):
    f = lib.qoq_rmsnorm_quantize_act
    assert f(A, A, 1e-5, 0, 128, A, A, A, NUL, NUL) == OK
    assert f(A, A, 1e-5, -1, 128, A, A, A, NUL, NUL) == ERR_SHAPE
    assert f(A, A, 1e-5, 4, 100, A, A, A, NUL, NUL) == ERR_SHAPE
    assert f(A, A, 1e-5, 4, 32768 + 128, A, A, A, NUL, NUL) == ERR_SHAPE  # row longer than the limit
    for eps in (0.0, -1e-5, float("inf"), float("nan")):
        assert f(A, A, eps, 4, 128, A, A, A, NUL, NUL) == ERR_SHAPE
    assert f(NUL, A, 1e-5, 4, 128, A, A, A, NUL, NUL) == ERR_NULL
    assert f(A, NUL, 1e-5, 4, 128, A, A, A, NUL, NUL) == ERR_NULL
    assert f(A, U, 1e-5, 4, 128, A, A, A, NUL, NUL) == ERR_ALIGN
    assert f(A, A, 1e-5, 4, 128, A, A, A, U, NUL) == ERR_ALIGN


def test_kv4_validation(lib):
    f = lib.qoq_kv4_smooth_scales
    assert f(A, 4, 8, 64, A, NUL) == ERR_SHAPE  # head dimension must be 128
    assert f(A, 4, 8, 128, NUL, NUL) == ERR_NULL
    assert f(U, 4, 8, 128, A, NUL) == ERR_ALIGN
    ap = lib.qoq_kv4_append
    def app(B=2, T=1, H=8, d=128, Tcap=32, t0=0, k=A):
        return ap(k, A, A, B, T, H, d, Tcap, t0, A, A, A, A, A, A, NUL)
    assert app(Tcap=30) == ERR_SHAPE  # Tcap a multiple of 16
    assert app(t0=32) == ERR_SHAPE  # past the capacity
    assert app(T=0) == OK
    assert app(k=NUL) == ERR_NULL
    assert app(k=U) == ERR_ALIGN
    w = lib.qoq_kv4_attention_workspace_bytes
    assert w(2, 32, 8, 128, 1536) > 0
    assert w(2, 24, 8, 128, 1536) == -1  # group of 3
    assert w(2, 128, 8, 128, 1536) == -1  # group of 16
    at = lib.qoq_kv4_decode_attention
    need = w(2, 32, 8, 128, 1536)
    def att(ws=A, wsb=need, lens=A):
        return at(A, A, A, A, A, A, A, A, lens, 2, 32, 8, 128, 1536, A, ws, wsb, NUL)
    assert att(ws=NUL) == ERR_NULL
    assert att(lens=NUL) == ERR_NULL
    assert att(wsb=need - 1) == ERR_WORKSPACE



# ---- checkpoint header ------------------------------------------------------
def _header(lib, fmt, N, K):
    h = qoq.BlobHeader()
    assert lib.qoq_blob_header_init(fmt, N, K, ctypes.byref(h)) == OK
    return h


def test_blob_header_layout_and_fields(lib):
    assert ctypes.sizeof(qoq.BlobHeader) == 64
    hdr = open(HEADER).read()
    ver = int(re.search(r"#define QOQ_ABI_VERSION (\d+)", hdr).group(1))
    h = _header(lib, 0, 6144, 4096)
    raw = bytes(h)
    assert raw[:4] == b"QPK1"
    assert (h.magic, h.abi_version, h.format, h.group) == (qoq.BLOB_MAGIC, ver, 0, 128)
    assert (h.n, h.k, h.blob_bytes, h.scale_bytes) == (6144, 4096, 6144 * 2048 + 6144 * 32, 2 * 6144)
    assert bytes(h.reserved) == bytes(16)
    assert _header(lib, 1, 16, 128).blob_bytes == 16 * 64 + 16
    assert _header(lib, qoq.FORMAT_W8A8, 32, 256).blob_bytes == 32 * 256
    assert lib.qoq_blob_header_check(ctypes.byref(h), 0, 6144, 4096) == OK


@pytest.mark.parametrize("field,value", [
    ("magic", 0x314B5052), ("abi_version", 5), ("format", 1), ("group", 64), ("n", 6160),
    ("k", 4224), ("blob_bytes", 6144 * 2048), ("scale_bytes", 6144)])
def test_blob_header_rejects_any_mismatch(lib, field, value):
    h = _header(lib, 0, 6144, 4096)
    setattr(h, field, value)
    assert lib.qoq_blob_header_check(ctypes.byref(h), 0, 6144, 4096) == ERR_HEADER


def test_blob_header_rejects_wrong_expectation_and_reserved_bytes(lib):
    h = _header(lib, 0, 6144, 4096)
    assert lib.qoq_blob_header_check(ctypes.byref(h), 1, 6144, 4096) == ERR_HEADER  # other mode
    assert lib.qoq_blob_header_check(ctypes.byref(h), 0, 6144, 8192) == ERR_HEADER  # other K
    assert lib.qoq_blob_header_check(ctypes.byref(h), 0, 4096, 4096) == ERR_HEADER  # other N
    h.reserved[7] = 1
    assert lib.qoq_blob_header_check(ctypes.byref(h), 0, 6144, 4096) == ERR_HEADER
    assert lib.qoq_blob_header_check(None, 0, 6144, 4096) == ERR_NULL
    assert lib.qoq_blob_header_init(0, 6144, 4096, None) == ERR_NULL
    assert lib.qoq_blob_header_init(3, 16, 128, ctypes.byref(h)) == ERR_MODE
    assert lib.qoq_blob_header_init(0, 15, 128, ctypes.byref(h)) == ERR_SHAPE
    assert lib.qoq_blob_header_init(0, 16, 100, ctypes.byref(h)) == ERR_SHAPE


def test_checkpoint_loader_refuses_mismatches(lib, tmp_path):
    """PackedWeight.load checks the header and the length before touching a
    device: a checkpoint for another shape or format, a truncated one or one
    from another ABI version is refused on the host."""
    N, K = 32, 256
    h = _header(lib, 0, N, K)
    body = bytes(h.blob_bytes) + bytes(h.scale_bytes)
    good = tmp_path / "w.qpk"
    good.write_bytes(bytes(h) + body)
    for mode, n, k in ((1, N, K), (0, N, 384), (0, 48, K), (qoq.W8A8, N, K)):
        with pytest.raises(qoq.QoQError):
            qoq.PackedWeight.load(str(good), mode, n, k, "cpu")
    short = tmp_path / "short.qpk"
    short.write_bytes(bytes(h) + body[:-1])
    with pytest.raises(qoq.QoQError):
        qoq.PackedWeight.load(str(short), 0, N, K, "cpu")
    h.abi_version -= 1
    old = tmp_path / "old.qpk"
    old.write_bytes(bytes(h) + body)
    with pytest.raises(qoq.QoQError):
        qoq.PackedWeight.load(str(old), 0, N, K, "cpu")
    pw = qoq.PackedWeight.load(str(good), 0, N, K, "cpu")  # a matching header loads
    assert pw.blob.numel() == N * K // 2 + N * K // 128 and pw.s_c.numel() == N
