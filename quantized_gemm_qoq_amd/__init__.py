"""QoQ W4A8 GEMM (and its W8A8 and W4A16 siblings) for AMD Instinct MI355X (gfx950).

Python binding of ``libqoq.so`` (the C ABI declared in ``include/qoq.h``). The
functions carry the C names and do argument marshalling only: every step of
the path runs in the library's HIP kernels. PyTorch provides the device memory
(tensors, whose ``data_ptr`` is passed) and the stream (the current stream of
the tensors' device). There is no fallback: if the library cannot be loaded,
or a call fails, a ``QoQError`` is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

MODE_G128 = 0
MODE_PER_CHANNEL = 1
GROUP = 128
MAX_K = 132096
MODES = {"g128": MODE_G128, "per_channel": MODE_PER_CHANNEL}
W8A8 = "w8a8"  # the INT8-weight sibling format (its own entry points)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqoq.so")

# Every entry point that include/qoq.h declares.
EXPORTED = (
    "qoq_abi_version",
    "qoq_status_str",
    "qoq_quantize_weights",
    "qoq_packed_bytes",
    "qoq_pack_weights",
    "qoq_unpack_weights",
    "qoq_act_bytes",
    "qoq_quantize_act",
    "qoq_gemm_workspace_bytes",
    "qoq_w4a8_gemm",
    "qoq_w8a8_quantize_weights",
    "qoq_w8a8_packed_bytes",
    "qoq_w8a8_pack_weights",
    "qoq_w8a8_gemm_workspace_bytes",
    "qoq_w8a8_gemm",
    "qoq_w4a16_gemm",
    "qoq_silu_mul_quantize_act",
    "qoq_rmsnorm_quantize_act",
    "qoq_silu_mul_workspace_bytes",
    "qoq_silu_mul_quantize_act_ws",
    "qoq_kv4_smooth_scales",
    "qoq_kv4_append",
    "qoq_kv4_attention_workspace_bytes",
    "qoq_kv4_decode_attention",
    "qoq_blob_header_init",
    "qoq_blob_header_check",
    "qoq_w4a8_gemm_noalloc",
)

FORMAT_W8A8 = 2  # format code of the W8A8 blob in a checkpoint header
BLOB_MAGIC = 0x314B5051


class BlobHeader(ctypes.Structure):
    """qoq_blob_header of include/qoq.h (64 bytes, little-endian, no padding)."""
    _fields_ = [("magic", ctypes.c_uint32), ("abi_version", ctypes.c_uint32),
                ("format", ctypes.c_uint32), ("group", ctypes.c_uint32),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("blob_bytes", ctypes.c_int64), ("scale_bytes", ctypes.c_int64),
                ("reserved", ctypes.c_uint8 * 16)]


class QoQError(RuntimeError):
    pass


_lock = threading.Lock()
_lib = None


def load_library():
    """Load libqoq.so (building it first if it has never been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            from . import build

            build.build()
        lib = ctypes.CDLL(LIB_PATH)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        sigs = {
            "qoq_abi_version": (I, []),
            "qoq_status_str": (ctypes.c_char_p, [I]),
            "qoq_quantize_weights": (I, [I, P, I64, I64, P, P, P, P, P]),
            "qoq_packed_bytes": (I64, [I, I64, I64]),
            "qoq_pack_weights": (I, [I, P, P, P, I64, I64, P, P]),
            "qoq_unpack_weights": (I, [I, P, I64, I64, P, P, P, P]),
            "qoq_act_bytes": (I64, [I64, I64]),
            "qoq_quantize_act": (I, [P, I64, I64, P, P, P, P]),
            "qoq_gemm_workspace_bytes": (I64, [I, I64, I64, I64]),
            "qoq_w4a8_gemm": (I, [I, P, P, P, P, P, I64, I64, I64, P, P, P, I64, P]),
            "qoq_w8a8_quantize_weights": (I, [P, I64, I64, P, P, P]),
            "qoq_w8a8_packed_bytes": (I64, [I64, I64]),
            "qoq_w8a8_pack_weights": (I, [P, I64, I64, P, P]),
            "qoq_w8a8_gemm_workspace_bytes": (I64, [I64, I64, I64]),
            "qoq_w8a8_gemm": (I, [P, P, P, P, I64, I64, I64, P, P, P, I64, P]),
            "qoq_w4a16_gemm": (I, [I, P, P, P, I64, I64, I64, P, P, P]),
            "qoq_silu_mul_quantize_act": (I, [P, I64, I64, P, P, P, P, P]),
            "qoq_rmsnorm_quantize_act": (I, [P, P, ctypes.c_float, I64, I64, P, P, P, P, P]),
            "qoq_silu_mul_workspace_bytes": (I64, [I64, I64]),
            "qoq_silu_mul_quantize_act_ws": (I, [P, I64, I64, P, P, P, P, P, I64, P]),
            "qoq_kv4_smooth_scales": (I, [P, I64, I64, I64, P, P]),
            "qoq_kv4_append": (I, [P, P, P, I64, I64, I64, I64, I64, I64, P, P, P, P, P, P, P]),
            "qoq_kv4_attention_workspace_bytes": (I64, [I64, I64, I64, I64, I64]),
            "qoq_kv4_decode_attention": (I, [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64,
                                             P, P, I64, P]),
            "qoq_blob_header_init": (I, [I, I64, I64, ctypes.POINTER(BlobHeader)]),
            "qoq_blob_header_check": (I, [ctypes.POINTER(BlobHeader), I, I64, I64]),
            "qoq_w4a8_gemm_noalloc": (I, [I, P, P, P, P, P, I64, I64, I64, P, P, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _mode(mode) -> int:
    if isinstance(mode, str):
        return MODES[mode]
    return int(mode)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, dtype, name: str, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise QoQError(f"{name} must live in GPU memory (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise QoQError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise QoQError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _check(status: int, name: str):
    if status != 0:
        msg = load_library().qoq_status_str(status).decode()
        raise QoQError(f"{name}: {msg} (status {status})")


def qoq_abi_version() -> int:
    return int(load_library().qoq_abi_version())


def qoq_status_str(status: int) -> str:
    return load_library().qoq_status_str(int(status)).decode()


def qoq_packed_bytes(mode, N: int, K: int) -> int:
    return int(load_library().qoq_packed_bytes(_mode(mode), int(N), int(K)))


def qoq_quantize_weights(mode, w: torch.Tensor, q=None, s_c=None, s_g=None, z=None):
    """W [N,K] fp16 -> (q uint8 [N,K], s_c fp16 [N], s_g uint8 [N,K/128] | None, z uint8)."""
    mode = _mode(mode)
    _need(w, torch.float16, "w")
    N, K = w.shape
    dev = w.device
    q = q if q is not None else torch.empty((N, K), dtype=torch.uint8, device=dev)
    s_c = s_c if s_c is not None else torch.empty((N,), dtype=torch.float16, device=dev)
    if mode == MODE_G128:
        G = K // GROUP
        s_g = s_g if s_g is not None else torch.empty((N, G), dtype=torch.uint8, device=dev)
        z = z if z is not None else torch.empty((N, G), dtype=torch.uint8, device=dev)
        _need(s_g, torch.uint8, "s_g", (N, G))
        _need(z, torch.uint8, "z", (N, G))
    else:
        s_g = None
        z = z if z is not None else torch.empty((N,), dtype=torch.uint8, device=dev)
        _need(z, torch.uint8, "z", (N,))
    _need(q, torch.uint8, "q", (N, K))
    _need(s_c, torch.float16, "s_c", (N,))
    st = load_library().qoq_quantize_weights(mode, _ptr(w), N, K, _ptr(q), _ptr(s_c), _ptr(s_g),
                                             _ptr(z), _stream(w))
    _check(st, "qoq_quantize_weights")
    return q, s_c, s_g, z


def qoq_pack_weights(mode, q: torch.Tensor, s_g: Optional[torch.Tensor], z: torch.Tensor,
                     blob: Optional[torch.Tensor] = None) -> torch.Tensor:
    mode = _mode(mode)
    _need(q, torch.uint8, "q")
    N, K = q.shape
    nbytes = qoq_packed_bytes(mode, N, K)
    if nbytes < 0:
        raise QoQError(f"qoq_pack_weights: unsupported shape N={N} K={K}")
    blob = blob if blob is not None else torch.empty((nbytes,), dtype=torch.uint8, device=q.device)
    _need(blob, torch.uint8, "blob", (nbytes,))
    _need(z, torch.uint8, "z")
    if s_g is not None:
        _need(s_g, torch.uint8, "s_g")
    st = load_library().qoq_pack_weights(mode, _ptr(q), _ptr(s_g), _ptr(z), N, K, _ptr(blob),
                                         _stream(q))
    _check(st, "qoq_pack_weights")
    return blob


def qoq_unpack_weights(mode, blob: torch.Tensor, N: int, K: int):
    mode = _mode(mode)
    _need(blob, torch.uint8, "blob")
    dev = blob.device
    q = torch.empty((N, K), dtype=torch.uint8, device=dev)
    if mode == MODE_G128:
        s_g = torch.empty((N, K // GROUP), dtype=torch.uint8, device=dev)
        z = torch.empty((N, K // GROUP), dtype=torch.uint8, device=dev)
    else:
        s_g = None
        z = torch.empty((N,), dtype=torch.uint8, device=dev)
    st = load_library().qoq_unpack_weights(mode, _ptr(blob), N, K, _ptr(q), _ptr(s_g), _ptr(z),
                                           _stream(blob))
    _check(st, "qoq_unpack_weights")
    return q, s_g, z


def qoq_act_bytes(M: int, K: int) -> int:
    return int(load_library().qoq_act_bytes(int(M), int(K)))


def qoq_quantize_act(x: torch.Tensor, xq=None, s_x=None, rowsum=None, want_rowsum: bool = True):
    """X [M,K] fp16 -> (xq, s_x fp16 [M], rowsum int32 [M] | None).

    xq is a flat int8 tensor of qoq_act_bytes(M, K) bytes in the packed tile
    order the GEMM reads (the layout is written out in include/qoq.h)."""
    _need(x, torch.float16, "x")
    M, K = x.shape
    dev = x.device
    nbytes = qoq_act_bytes(M, K)
    if nbytes < 0:
        raise QoQError(f"qoq_quantize_act: unsupported shape M={M} K={K}")
    xq = xq if xq is not None else torch.empty((nbytes,), dtype=torch.int8, device=dev)
    s_x = s_x if s_x is not None else torch.empty((M,), dtype=torch.float16, device=dev)
    if rowsum is None and want_rowsum:
        rowsum = torch.empty((M,), dtype=torch.int32, device=dev)
    _need(xq, torch.int8, "xq", (nbytes,))
    _need(s_x, torch.float16, "s_x", (M,))
    if rowsum is not None:
        _need(rowsum, torch.int32, "rowsum", (M,))
    st = load_library().qoq_quantize_act(_ptr(x), M, K, _ptr(xq), _ptr(s_x), _ptr(rowsum),
                                         _stream(x))
    _check(st, "qoq_quantize_act")
    return xq, s_x, rowsum


def qoq_silu_mul_quantize_act(gate_up: torch.Tensor, xq=None, s_x=None, rowsum=None,
                              want_rowsum: bool = True, h=None, workspace="auto"):
    """gate_up [M, 2I] fp16 -> (xq, s_x, rowsum | None) of h = f16(SiLU(gate) * up),
    gate = columns 0..I-1, up = columns I..2I-1; the same outputs as
    qoq_quantize_act(h). h (fp16 [M, I]) is written too when given.
    workspace: "auto" allocates the split-row workspace when the shape uses one,
    None runs the one-pass kernels, or a uint8 device tensor."""
    _need(gate_up, torch.float16, "gate_up")
    M, I2 = gate_up.shape
    if I2 % 2:
        raise QoQError("gate_up must have an even number of columns")
    I = I2 // 2
    dev = gate_up.device
    nbytes = qoq_act_bytes(M, I)
    if nbytes < 0:
        raise QoQError(f"qoq_silu_mul_quantize_act: unsupported shape M={M} I={I}")
    xq = xq if xq is not None else torch.empty((nbytes,), dtype=torch.int8, device=dev)
    s_x = s_x if s_x is not None else torch.empty((M,), dtype=torch.float16, device=dev)
    if rowsum is None and want_rowsum:
        rowsum = torch.empty((M,), dtype=torch.int32, device=dev)
    _need(xq, torch.int8, "xq", (nbytes,))
    _need(s_x, torch.float16, "s_x", (M,))
    if rowsum is not None:
        _need(rowsum, torch.int32, "rowsum", (M,))
    if h is not None:
        _need(h, torch.float16, "h", (M, I))
    lib = load_library()
    if isinstance(workspace, str):
        need = int(lib.qoq_silu_mul_workspace_bytes(M, I))
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev) if need > 0 else None
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib.qoq_silu_mul_quantize_act_ws(_ptr(gate_up), M, I, _ptr(xq), _ptr(s_x), _ptr(rowsum),
                                          _ptr(h), _ptr(workspace), ws_bytes, _stream(gate_up))
    _check(st, "qoq_silu_mul_quantize_act")
    return xq, s_x, rowsum


def qoq_rmsnorm_quantize_act(x: torch.Tensor, gamma: torch.Tensor, eps: float, xq=None, s_x=None,
                             rowsum=None, want_rowsum: bool = True, y=None):
    """x [M, K] fp16, gamma [K] fp16, eps > 0 -> (xq, s_x, rowsum | None) of
    y = f16((x * r) * gamma), r = 1 / sqrt(mean(x^2) + eps) (the exact sum of
    squares); the same outputs as qoq_quantize_act(y). y (fp16 [M, K]) is
    written too when given."""
    _need(x, torch.float16, "x")
    M, K = x.shape
    _need(gamma, torch.float16, "gamma", (K,))
    dev = x.device
    nbytes = qoq_act_bytes(M, K)
    if nbytes < 0:
        raise QoQError(f"qoq_rmsnorm_quantize_act: unsupported shape M={M} K={K}")
    xq = xq if xq is not None else torch.empty((nbytes,), dtype=torch.int8, device=dev)
    s_x = s_x if s_x is not None else torch.empty((M,), dtype=torch.float16, device=dev)
    if rowsum is None and want_rowsum:
        rowsum = torch.empty((M,), dtype=torch.int32, device=dev)
    _need(xq, torch.int8, "xq", (nbytes,))
    _need(s_x, torch.float16, "s_x", (M,))
    if rowsum is not None:
        _need(rowsum, torch.int32, "rowsum", (M,))
    if y is not None:
        _need(y, torch.float16, "y", (M, K))
    st = load_library().qoq_rmsnorm_quantize_act(_ptr(x), _ptr(gamma), float(eps), M, K, _ptr(xq),
                                                 _ptr(s_x), _ptr(rowsum), _ptr(y), _stream(x))
    _check(st, "qoq_rmsnorm_quantize_act")
    return xq, s_x, rowsum


def qoq_gemm_workspace_bytes(mode, M: int, N: int, K: int) -> int:
    return int(load_library().qoq_gemm_workspace_bytes(_mode(mode), int(M), int(N), int(K)))


_workspaces = {}
_retired = []  # superseded workspaces: kept alive, a captured graph may still use them


def gemm_workspace(mode, M: int, N: int, K: int, device) -> Optional[torch.Tensor]:
    """The shared workspace of the device's current stream when the plan for
    this shape uses one (split-K partial sums), else None. ``mode`` is a W4
    mode or ``"w8a8"``.

    One workspace per (device, stream) serves every call on that stream that
    does not bring its own; calls on different streams never share one. It
    only grows: a workspace replaced by a larger one is kept alive until the
    process ends, so a HIP graph captured with it replays on valid memory."""
    if mode == W8A8:
        need = qoq_w8a8_gemm_workspace_bytes(M, N, K)
    else:
        need = qoq_gemm_workspace_bytes(mode, M, N, K)
    if need <= 0:
        return None
    dev = torch.device(device)
    index = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (index, torch.cuda.current_stream(index).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        if ws is not None:
            _retired.append(ws)
        ws = torch.zeros((max(need, 1 << 20),), dtype=torch.uint8, device=torch.device("cuda", index))
        _workspaces[key] = ws
    return ws


def qoq_w4a8_gemm(mode, xq: torch.Tensor, s_x: torch.Tensor, rowsum: Optional[torch.Tensor],
                  blob: torch.Tensor, s_c: torch.Tensor, N: int, y=None, acc_out=None,
                  workspace="auto", K: Optional[int] = None):
    """Y [M,N] fp16 = rescale(sum_k xq * unpack(blob)); acc_out (int32 [M,N]) optional.

    xq: packed activations from qoq_quantize_act (M is the length of s_x).
    workspace: "auto" (the shared workspace of the current stream), None (a
    plan that needs none) or a uint8 tensor of qoq_gemm_workspace_bytes()."""
    mode = _mode(mode)
    _need(xq, torch.int8, "xq")
    _need(s_x, torch.float16, "s_x")
    M = s_x.numel()
    dev = xq.device
    mp = (M + 15) // 16 * 16
    if K is None:
        if mp == 0:
            raise QoQError("qoq_w4a8_gemm: K must be given when M == 0")
        K = xq.numel() // mp
    if xq.numel() != mp * K:
        raise QoQError(f"xq has {xq.numel()} bytes, expected {mp} x {K}")
    _need(s_c, torch.float16, "s_c", (N,))
    _need(blob, torch.uint8, "blob")
    if rowsum is not None:
        _need(rowsum, torch.int32, "rowsum", (M,))
    y = y if y is not None else torch.empty((M, N), dtype=torch.float16, device=dev)
    _need(y, torch.float16, "y", (M, N))
    if acc_out is not None:
        _need(acc_out, torch.int32, "acc_out", (M, N))
    nbytes = qoq_packed_bytes(mode, N, K)
    if M and N and blob.numel() != nbytes:
        raise QoQError(f"blob has {blob.numel()} bytes, expected {nbytes}")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a tensor")
        workspace = gemm_workspace(mode, M, N, K, dev) if M and N else None
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    st = load_library().qoq_w4a8_gemm(mode, _ptr(xq), _ptr(s_x), _ptr(rowsum), _ptr(blob),
                                      _ptr(s_c), M, N, K, _ptr(y), _ptr(acc_out), _ptr(workspace),
                                      ws_bytes, _stream(xq))
    _check(st, "qoq_w4a8_gemm")
    return y


# ---- W8A8 sibling ---------------------------------------------------------

def qoq_w8a8_packed_bytes(N: int, K: int) -> int:
    return int(load_library().qoq_w8a8_packed_bytes(int(N), int(K)))


def qoq_w8a8_quantize_weights(w: torch.Tensor, q=None, s_c=None):
    """W [N,K] fp16 -> (q int8 [N,K], s_c fp16 [N]), per-channel symmetric INT8."""
    _need(w, torch.float16, "w")
    N, K = w.shape
    dev = w.device
    q = q if q is not None else torch.empty((N, K), dtype=torch.int8, device=dev)
    s_c = s_c if s_c is not None else torch.empty((N,), dtype=torch.float16, device=dev)
    _need(q, torch.int8, "q", (N, K))
    _need(s_c, torch.float16, "s_c", (N,))
    st = load_library().qoq_w8a8_quantize_weights(_ptr(w), N, K, _ptr(q), _ptr(s_c), _stream(w))
    _check(st, "qoq_w8a8_quantize_weights")
    return q, s_c


def qoq_w8a8_pack_weights(q: torch.Tensor, blob: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(q, torch.int8, "q")
    N, K = q.shape
    nbytes = qoq_w8a8_packed_bytes(N, K)
    if nbytes < 0:
        raise QoQError(f"qoq_w8a8_pack_weights: unsupported shape N={N} K={K}")
    blob = blob if blob is not None else torch.empty((nbytes,), dtype=torch.uint8, device=q.device)
    _need(blob, torch.uint8, "blob", (nbytes,))
    st = load_library().qoq_w8a8_pack_weights(_ptr(q), N, K, _ptr(blob), _stream(q))
    _check(st, "qoq_w8a8_pack_weights")
    return blob


def qoq_w8a8_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load_library().qoq_w8a8_gemm_workspace_bytes(int(M), int(N), int(K)))


def qoq_w8a8_gemm(xq: torch.Tensor, s_x: torch.Tensor, blob: torch.Tensor, s_c: torch.Tensor,
                  N: int, y=None, acc_out=None, workspace="auto", K: Optional[int] = None):
    """Y [M,N] fp16 = rescale(sum_k xq * q); acc_out (int32 [M,N]) optional.

    Arguments as for qoq_w4a8_gemm, with blob from qoq_w8a8_pack_weights."""
    _need(xq, torch.int8, "xq")
    _need(s_x, torch.float16, "s_x")
    M = s_x.numel()
    dev = xq.device
    mp = (M + 15) // 16 * 16
    if K is None:
        if mp == 0:
            raise QoQError("qoq_w8a8_gemm: K must be given when M == 0")
        K = xq.numel() // mp
    if xq.numel() != mp * K:
        raise QoQError(f"xq has {xq.numel()} bytes, expected {mp} x {K}")
    _need(s_c, torch.float16, "s_c", (N,))
    _need(blob, torch.uint8, "blob")
    y = y if y is not None else torch.empty((M, N), dtype=torch.float16, device=dev)
    _need(y, torch.float16, "y", (M, N))
    if acc_out is not None:
        _need(acc_out, torch.int32, "acc_out", (M, N))
    nbytes = qoq_w8a8_packed_bytes(N, K)
    if M and N and blob.numel() != nbytes:
        raise QoQError(f"blob has {blob.numel()} bytes, expected {nbytes}")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a tensor")
        workspace = gemm_workspace(W8A8, M, N, K, dev) if M and N else None
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    st = load_library().qoq_w8a8_gemm(_ptr(xq), _ptr(s_x), _ptr(blob), _ptr(s_c), M, N, K,
                                      _ptr(y), _ptr(acc_out), _ptr(workspace), ws_bytes,
                                      _stream(xq))
    _check(st, "qoq_w8a8_gemm")
    return y


# ---- W4A16 sibling --------------------------------------------------------

def qoq_w4a16_gemm(mode, x: torch.Tensor, blob: torch.Tensor, s_c: torch.Tensor, N: int,
                   y=None, acc_out=None):
    """Y [M,N] fp16 = f16(s_c * sum_k x * W8^) with FP16 x [M,K] (not quantized)
    and the W4 blob of qoq_pack_weights; acc_out (float32 [M,N]) optional."""
    mode = _mode(mode)
    _need(x, torch.float16, "x")
    M, K = x.shape
    dev = x.device
    _need(s_c, torch.float16, "s_c", (N,))
    _need(blob, torch.uint8, "blob")
    y = y if y is not None else torch.empty((M, N), dtype=torch.float16, device=dev)
    _need(y, torch.float16, "y", (M, N))
    if acc_out is not None:
        _need(acc_out, torch.float32, "acc_out", (M, N))
    nbytes = qoq_packed_bytes(mode, N, K)
    if M and N and blob.numel() != nbytes:
        raise QoQError(f"blob has {blob.numel()} bytes, expected {nbytes}")
    st = load_library().qoq_w4a16_gemm(mode, _ptr(x), _ptr(blob), _ptr(s_c), M, N, K, _ptr(y),
                                       _ptr(acc_out), _stream(x))
    _check(st, "qoq_w4a16_gemm")
    return y


# ---- KV4 decode attention with SmoothAttention ------------------------------

HEAD_DIM = 128


def qoq_kv4_smooth_scales(k_calib: torch.Tensor) -> torch.Tensor:
    """Calibration keys [T, H, 128] fp16 -> lambda [H, 128] fp16 (alpha = 0.5)."""
    _need(k_calib, torch.float16, "k_calib")
    T, H, d = k_calib.shape
    lam = torch.empty((H, d), dtype=torch.float16, device=k_calib.device)
    st = load_library().qoq_kv4_smooth_scales(_ptr(k_calib), T, H, d, _ptr(lam), _stream(k_calib))
    _check(st, "qoq_kv4_smooth_scales")
    return lam


class KV4Cache:
    """A KV4 cache of B sequences x H heads x Tcap tokens (layout in include/qoq.h)."""

    def __init__(self, B: int, H: int, Tcap: int, device, lam: torch.Tensor):
        if Tcap % 16:
            raise QoQError("Tcap must be a multiple of 16")
        self.B, self.H, self.Tcap = B, H, Tcap
        self.lam = _need(lam, torch.float16, "lambda", (H, HEAD_DIM))
        dev = torch.device(device)
        self.kq = torch.zeros((B, H, Tcap, HEAD_DIM // 2), dtype=torch.uint8, device=dev)
        self.vq = torch.zeros((B, H, Tcap // 16, HEAD_DIM // 2, 16), dtype=torch.uint8, device=dev)
        self.ks = torch.zeros((B, H, Tcap), dtype=torch.float16, device=dev)
        self.vs = torch.zeros((B, H, Tcap), dtype=torch.float16, device=dev)
        self.kz = torch.zeros((B, H, Tcap), dtype=torch.uint8, device=dev)
        self.vz = torch.zeros((B, H, Tcap), dtype=torch.uint8, device=dev)

    def append(self, k: torch.Tensor, v: torch.Tensor, t0: int):
        """Quantize k, v [B, T, H, 128] fp16 into positions t0 .. t0+T-1."""
        _need(k, torch.float16, "k")
        _need(v, torch.float16, "v", tuple(k.shape))
        B, T, H, d = k.shape
        st = load_library().qoq_kv4_append(_ptr(k), _ptr(v), _ptr(self.lam), B, T, H, d, self.Tcap,
                                           t0, _ptr(self.kq), _ptr(self.ks), _ptr(self.kz),
                                           _ptr(self.vq), _ptr(self.vs), _ptr(self.vz), _stream(k))
        _check(st, "qoq_kv4_append")

    def attention(self, q: torch.Tensor, lens: torch.Tensor, o=None, workspace=None):
        """One query token per sequence: q [B, Hq, 128] fp16, lens int32 [B] (device)
        -> o [B, Hq, 128] fp16."""
        _need(q, torch.float16, "q")
        _need(lens, torch.int32, "lens", (self.B,))
        B, Hq, d = q.shape
        need = int(load_library().qoq_kv4_attention_workspace_bytes(B, Hq, self.H, d, self.Tcap))
        if need < 0:
            raise QoQError(f"qoq_kv4_decode_attention: unsupported shape B={B} Hq={Hq} H={self.H}")
        if workspace is None:
            workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
        o = o if o is not None else torch.empty((B, Hq, d), dtype=torch.float16, device=q.device)
        _need(o, torch.float16, "o", (B, Hq, d))
        st = load_library().qoq_kv4_decode_attention(
            _ptr(q), _ptr(self.lam), _ptr(self.kq), _ptr(self.ks), _ptr(self.kz), _ptr(self.vq),
            _ptr(self.vs), _ptr(self.vz), _ptr(lens), B, Hq, self.H, d, self.Tcap, _ptr(o),
            _ptr(workspace), workspace.numel(), _stream(q))
        _check(st, "qoq_kv4_decode_attention")
        return o


class PackedWeight:
    """A weight matrix quantized and packed once (offline), kept resident.

    ``mode``: ``"g128"``, ``"per_channel"`` (W4A8) or ``"w8a8"`` (INT8 weights)."""

    def __init__(self, mode, w: torch.Tensor):
        self.mode = W8A8 if mode == W8A8 else _mode(mode)
        self.N, self.K = w.shape
        if self.mode == W8A8:
            q, self.s_c = qoq_w8a8_quantize_weights(w)
            self.blob = qoq_w8a8_pack_weights(q)
        else:
            q, self.s_c, s_g, z = qoq_quantize_weights(self.mode, w)
            self.blob = qoq_pack_weights(self.mode, q, s_g, z)

    def forward(self, x: torch.Tensor, y=None) -> torch.Tensor:
        """Per-call path: per-token INT8 quantization of x, then the GEMM."""
        xq, s_x, rowsum = qoq_quantize_act(x, want_rowsum=self.mode == MODE_PER_CHANNEL)
        if self.mode == W8A8:
            return qoq_w8a8_gemm(xq, s_x, self.blob, self.s_c, self.N, y=y, K=self.K)
        return qoq_w4a8_gemm(self.mode, xq, s_x, rowsum, self.blob, self.s_c, self.N, y=y,
                             K=self.K)

    def _format(self) -> int:
        return FORMAT_W8A8 if self.mode == W8A8 else int(self.mode)

    def save(self, path: str) -> None:
        """Write the checkpoint: the 64-byte qoq_blob_header, the blob, then s_c."""
        h = BlobHeader()
        _check(load_library().qoq_blob_header_init(self._format(), self.N, self.K, ctypes.byref(h)),
               "qoq_blob_header_init")
        with open(path, "wb") as f:
            f.write(bytes(h))
            f.write(self.blob.cpu().numpy().tobytes())
            f.write(self.s_c.cpu().view(torch.int16).numpy().tobytes())

    @classmethod
    def load(cls, path: str, mode, N: int, K: int, device) -> "PackedWeight":
        """Read a checkpoint written by save(), refusing (QoQError) one whose
        header does not describe a blob of this format and shape, or whose
        length does not match the header."""
        fmt = FORMAT_W8A8 if mode == W8A8 else _mode(mode)
        with open(path, "rb") as f:
            raw = f.read()
        if len(raw) < ctypes.sizeof(BlobHeader):
            raise QoQError(f"{path}: shorter than a checkpoint header")
        h = BlobHeader.from_buffer_copy(raw[:ctypes.sizeof(BlobHeader)])
        _check(load_library().qoq_blob_header_check(ctypes.byref(h), fmt, int(N), int(K)),
               f"checkpoint {path}")
        off = ctypes.sizeof(BlobHeader)
        if len(raw) != off + h.blob_bytes + h.scale_bytes:
            raise QoQError(f"{path}: {len(raw)} bytes, the header describes "
                           f"{off + h.blob_bytes + h.scale_bytes}")
        self = cls.__new__(cls)
        self.mode = W8A8 if mode == W8A8 else fmt
        self.N, self.K = int(N), int(K)
        blob = torch.frombuffer(bytearray(raw[off:off + h.blob_bytes]), dtype=torch.uint8)
        sc = torch.frombuffer(bytearray(raw[off + h.blob_bytes:]), dtype=torch.int16)
        self.blob = blob.to(device)
        self.s_c = sc.view(torch.float16).to(device)
        return self

    def forward_fp16(self, x: torch.Tensor, y=None) -> torch.Tensor:
        """The W4A16 sibling on the same 4-bit weights: FP16 x, no quantization."""
        if self.mode == W8A8:
            raise QoQError("forward_fp16 needs 4-bit weights")
        return qoq_w4a16_gemm(self.mode, x, self.blob, self.s_c, self.N, y=y)
