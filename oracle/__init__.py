"""CPU oracle for the QoQ W4A8 GEMM path (QServe, arXiv 2405.04532).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product path (the
HIP library under ``quantized_gemm_qoq_amd``) never imports it, and the two share
no code: the oracle is plain C in ``qoq_oracle.c``, loaded here through ctypes,
plus numpy library-product forms of its contractions for full-size shapes
(``gemm_matmul`` and its siblings), each pinned against the C loops.

Every function takes and returns numpy arrays. FP16 values travel as their raw
binary16 bits (``uint16``). What each function computes, and the passage of the
pages it follows, is stated beside it in ``qoq_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

MODE_G128 = 0
MODE_PER_CHANNEL = 1
GROUP = 128

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qoq_oracle.c")
_LIB = os.path.join(_HERE, "libqoq_oracle.so")
# A prebuilt copy of the same source to load instead (the sanitizer test
# builds one with AddressSanitizer and UndefinedBehaviorSanitizer).
_LIB_OVERRIDE = os.environ.get("QOQ_ORACLE_LIB")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if _LIB_OVERRIDE:
                lib = ctypes.CDLL(_LIB_OVERRIDE)
            else:
                build()
                lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            I = ctypes.c_int
            sigs = {
                "orc_f16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
                "orc_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
                "orc_num_threads": (I, []),
                "orc_quantize_act": (I, [P, I64, I64, P, P, P]),
                "orc_quantize_weights_g128": (I, [P, I64, I64, P, P, P, P, P]),
                "orc_quantize_weights_pc": (I, [P, I64, I64, P, P, P]),
                "orc_dequantize_weights": (I, [I, P, P, P, P, I64, I64, P]),
                "orc_packed_bytes": (I64, [I, I64, I64]),
                "orc_pack": (I, [I, P, P, P, I64, I64, P]),
                "orc_gemm": (I, [I, P, P, P, P, I64, I64, I64, P]),
                "orc_gemm_points": (I, [I, P, P, P, P, I64, I64, I64, I64, P, P, P]),
                "orc_epilogue": (I, [P, P, P, I64, I64, P]),
                "orc_epilogue_points": (I, [P, P, P, I64, P, P, P]),
                "orc_f32_to_f16_array": (None, [P, I64, P]),
                "orc_act_bytes": (I64, [I64, I64]),
                "orc_pack_act": (I, [P, I64, I64, P]),
                "orc_f16_to_f64_array": (None, [P, I64, P]),
                "orc_quantize_weights_w8": (I, [P, I64, I64, P, P]),
                "orc_w8_packed_bytes": (I64, [I64, I64]),
                "orc_pack_w8": (I, [P, I64, I64, P]),
                "orc_gemm_w8": (I, [P, P, I64, I64, I64, P]),
                "orc_gemm_w8_points": (I, [P, P, I64, I64, I64, I64, P, P, P]),
                "orc_gemm_w4a16": (I, [I, P, P, P, P, P, I64, I64, I64, P, P]),
                "orc_gemm_w4a16_points": (I, [I, P, P, P, P, P, I64, I64, I64, I64, P, P, P, P]),
                "orc_exp_f32_array": (None, [P, I64, P]),
                "orc_silu_mul": (I, [P, I64, I64, P]),
                "orc_kv4_smooth_scales": (I, [P, I64, I64, I64, P]),
                "orc_kv4_quantize": (I, [P, P, P, I64, I64, I64, I64, I64, P, P, P, P, P, P]),
                "orc_kv4_decode_attention": (I, [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64,
                                                 I64, P]),
                "orc_rmsnorm": (I, [P, P, ctypes.c_float, I64, I64, P, P]),
            }
            for name, (res, args) in sigs.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def num_threads() -> int:
    return _load().orc_num_threads()


def f32_to_f16_bits(values) -> np.ndarray:
    """binary32 -> binary16 bits (RNE) through the oracle's own conversion."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32).ravel())
    out = np.empty(v.size, np.uint16)
    _load().orc_f32_to_f16_array(_p(v), v.size, _p(out))
    return out


def f16_bits_to_f64(bits) -> np.ndarray:
    """binary16 bits -> exact value, through the oracle's own decoding."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16).ravel())
    out = np.empty(b.size, np.float64)
    _load().orc_f16_to_f64_array(_p(b), b.size, _p(out))
    return out


def quantize_act(x_bits):
    """Per-token INT8: returns (xq int8 [M,K], s_x uint16 [M], rowsum int32 [M])."""
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    s_x = np.empty(M, np.uint16)
    rowsum = np.empty(M, np.int32)
    _check(_load().orc_quantize_act(_p(x), M, K, _p(xq), _p(s_x), _p(rowsum)), "quantize_act")
    return xq, s_x, rowsum


def act_bytes(M, K) -> int:
    return int(_load().orc_act_bytes(M, K))


def pack_act(xq):
    """Row-major INT8 activations [M,K] -> the packed tile order (flat int8)."""
    xq = _c(xq, np.int8)
    M, K = xq.shape
    n = act_bytes(M, K)
    if n < 0:
        raise ValueError("shape not packable")
    out = np.empty(n, np.int8)
    _check(_load().orc_pack_act(_p(xq), M, K, _p(out)), "pack_act")
    return out


def quantize_weights(mode, w_bits, want_w8=False):
    """Progressive (g128) or per-channel W4 quantization.

    Returns dict with s_c uint16 [N], q uint8 [N,K], z uint8 ([N,G] or [N]),
    s_g uint8 [N,G] (g128 only) and, when asked, w8 int8 [N,K] (g128 only).
    """
    w = _c(w_bits, np.uint16)
    N, K = w.shape
    lib = _load()
    s_c = np.empty(N, np.uint16)
    q = np.empty((N, K), np.uint8)
    if mode == MODE_G128:
        G = K // GROUP
        s_g = np.empty((N, G), np.uint8)
        z = np.empty((N, G), np.uint8)
        w8 = np.empty((N, K), np.int8) if want_w8 else None
        _check(lib.orc_quantize_weights_g128(_p(w), N, K, _p(s_c), _p(q), _p(s_g), _p(z), _p(w8)),
               "quantize_weights_g128")
        out = {"s_c": s_c, "q": q, "s_g": s_g, "z": z}
        if want_w8:
            out["w8"] = w8
        return out
    if mode == MODE_PER_CHANNEL:
        z = np.empty(N, np.uint8)
        _check(lib.orc_quantize_weights_pc(_p(w), N, K, _p(s_c), _p(q), _p(z)),
               "quantize_weights_pc")
        return {"s_c": s_c, "q": q, "z": z, "s_g": None}
    raise ValueError("bad mode")


def dequantize_weights(mode, s_c, q, s_g, z):
    q = _c(q, np.uint8)
    N, K = q.shape
    out = np.empty((N, K), np.float64)
    sg = None if s_g is None else _c(s_g, np.uint8)
    _check(_load().orc_dequantize_weights(mode, _p(_c(s_c, np.uint16)), _p(q), _p(sg),
                                          _p(_c(z, np.uint8)), N, K, _p(out)),
           "dequantize_weights")
    return out


def packed_bytes(mode, N, K) -> int:
    return int(_load().orc_packed_bytes(mode, N, K))


def pack(mode, q, s_g, z):
    q = _c(q, np.uint8)
    N, K = q.shape
    nbytes = packed_bytes(mode, N, K)
    if nbytes < 0:
        raise ValueError("shape not packable")
    blob = np.empty(nbytes, np.uint8)
    sg = None if s_g is None else _c(s_g, np.uint8)
    _check(_load().orc_pack(mode, _p(q), _p(sg), _p(_c(z, np.uint8)), N, K, _p(blob)), "pack")
    return blob


def gemm(mode, xq, q, s_g, z):
    """Exact accumulator acc int32 [M,N]."""
    xq = _c(xq, np.int8)
    q = _c(q, np.uint8)
    M, K = xq.shape
    N = q.shape[0]
    acc = np.empty((M, N), np.int32)
    sg = None if s_g is None else _c(s_g, np.uint8)
    _check(_load().orc_gemm(mode, _p(xq), _p(q), _p(sg), _p(_c(z, np.uint8)), M, N, K, _p(acc)),
           "gemm")
    return acc


def gemm_points(mode, xq, q, s_g, z, ms, ns):
    xq = _c(xq, np.int8)
    q = _c(q, np.uint8)
    M, K = xq.shape
    N = q.shape[0]
    ms = _c(np.asarray(ms, np.int64), np.int64)
    ns = _c(np.asarray(ns, np.int64), np.int64)
    acc = np.empty(len(ms), np.int32)
    sg = None if s_g is None else _c(s_g, np.uint8)
    _check(_load().orc_gemm_points(mode, _p(xq), _p(q), _p(sg), _p(_c(z, np.uint8)), M, N, K,
                                   len(ms), _p(ms), _p(ns), _p(acc)), "gemm_points")
    return acc


def weights_int(mode, q, s_g, z):
    """The integer weights the accumulator contracts, [N, K] int32: g128
    (q - z[n, k/128]) * s_g[n, k/128], per-channel q - z[n] (the same values
    orc_gemm forms row by row)."""
    q = _c(q, np.uint8).astype(np.int32)
    if mode == MODE_G128:
        zz = np.repeat(_c(z, np.uint8).astype(np.int32), GROUP, axis=1)
        ss = np.repeat(_c(s_g, np.uint8).astype(np.int32), GROUP, axis=1)
        return (q - zz) * ss
    if mode == MODE_PER_CHANNEL:
        return q - _c(z, np.uint8).astype(np.int32)[:, None]
    raise ValueError("bad mode")


# Output channels per library product in the matmul forms below (bounds the
# float64 copy of the weights to a few hundred MB).
_CHANNEL_SLICE = 2048


def _exact_int_matmul(xf, wf):
    """xf [M,K] @ wf [n,K]^T in float64 for integer-valued operands, returned
    as int32 (an error if a sum leaves the int32 range, as in orc_gemm). Exact:
    every product and every partial sum is an integer of magnitude at most
    max_m sum_k |x[m,k]| * max |w|, checked below 2^53, so float64 holds every
    intermediate exactly whatever order the library adds them in."""
    if xf.size and wf.size and np.abs(xf).sum(axis=1).max() * np.abs(wf).max() >= 2.0**53:
        raise OverflowError("partial sums could exceed 2^53")
    r = xf @ wf.T
    if r.size and (r.max() > 2.0**31 - 1 or r.min() < -(2.0**31)):
        raise OverflowError("accumulator outside int32")
    return r.astype(np.int32)


def gemm_matmul(mode, xq, q, s_g, z):
    """The accumulator of gemm() [M, N] int32, computed as library matrix
    products (numpy float64, one per slice of output channels) of Xq and the
    integer weights of weights_int(): the definition acc = Xq . W8^T with a
    matmul as its one step, exact as _exact_int_matmul states. For shapes the C
    loops of gemm() take minutes over."""
    xf = _c(xq, np.int8).astype(np.float64)
    q = _c(q, np.uint8)
    M, N = xf.shape[0], q.shape[0]
    acc = np.empty((M, N), np.int32)
    for n0 in range(0, N, _CHANNEL_SLICE):
        n1 = min(N, n0 + _CHANNEL_SLICE)
        sg = None if s_g is None else np.asarray(s_g)[n0:n1]
        zz = np.asarray(z)[n0:n1]
        acc[:, n0:n1] = _exact_int_matmul(xf, weights_int(mode, q[n0:n1], sg, zz).astype(np.float64))
    return acc


def epilogue(acc, s_x, s_c):
    """Y = acc * s_x * s_c in fp64 (exact), shape [M,N]."""
    acc = _c(acc, np.int32)
    M, N = acc.shape
    y = np.empty((M, N), np.float64)
    _check(_load().orc_epilogue(_p(acc), _p(_c(s_x, np.uint16)), _p(_c(s_c, np.uint16)), M, N,
                                _p(y)), "epilogue")
    return y


def epilogue_points(acc, s_x, s_c, ms, ns):
    acc = _c(acc, np.int32)
    ms = _c(np.asarray(ms, np.int64), np.int64)
    ns = _c(np.asarray(ns, np.int64), np.int64)
    y = np.empty(len(ms), np.float64)
    _check(_load().orc_epilogue_points(_p(acc), _p(_c(s_x, np.uint16)), _p(_c(s_c, np.uint16)),
                                       len(ms), _p(ms), _p(ns), _p(y)), "epilogue_points")
    return y


def forward(mode, x_bits, w_bits):
    """The whole path on the host: quantize both sides, contract, rescale."""
    xq, s_x, rowsum = quantize_act(x_bits)
    wq = quantize_weights(mode, w_bits)
    acc = gemm(mode, xq, wq["q"], wq["s_g"], wq["z"])
    y = epilogue(acc, s_x, wq["s_c"])
    return {"xq": xq, "s_x": s_x, "rowsum": rowsum, "acc": acc, "y": y, **wq}


# --- W8A8 sibling: per-channel symmetric INT8 weights (reading R13) ---------

def quantize_weights_w8(w_bits):
    """Returns (s_c uint16 [N], q int8 [N,K])."""
    w = _c(w_bits, np.uint16)
    N, K = w.shape
    s_c = np.empty(N, np.uint16)
    q = np.empty((N, K), np.int8)
    _check(_load().orc_quantize_weights_w8(_p(w), N, K, _p(s_c), _p(q)), "quantize_weights_w8")
    return s_c, q


def w8_packed_bytes(N, K) -> int:
    return int(_load().orc_w8_packed_bytes(N, K))


def pack_w8(q):
    q = _c(q, np.int8)
    N, K = q.shape
    n = w8_packed_bytes(N, K)
    if n < 0:
        raise ValueError("shape not packable")
    blob = np.empty(n, np.uint8)
    _check(_load().orc_pack_w8(_p(q), N, K, _p(blob)), "pack_w8")
    return blob


def gemm_w8(xq, q):
    """Exact accumulator acc int32 [M,N] = Xq . q^T."""
    xq = _c(xq, np.int8)
    q = _c(q, np.int8)
    M, K = xq.shape
    N = q.shape[0]
    acc = np.empty((M, N), np.int32)
    _check(_load().orc_gemm_w8(_p(xq), _p(q), M, N, K, _p(acc)), "gemm_w8")
    return acc


def gemm_w8_points(xq, q, ms, ns):
    xq = _c(xq, np.int8)
    q = _c(q, np.int8)
    M, K = xq.shape
    N = q.shape[0]
    ms = _c(np.asarray(ms, np.int64), np.int64)
    ns = _c(np.asarray(ns, np.int64), np.int64)
    acc = np.empty(len(ms), np.int32)
    _check(_load().orc_gemm_w8_points(_p(xq), _p(q), M, N, K, len(ms), _p(ms), _p(ns), _p(acc)),
           "gemm_w8_points")
    return acc


def gemm_w8_matmul(xq, q):
    """The accumulator of gemm_w8() [M, N] int32 as library matrix products in
    float64 (exact, as for gemm_matmul)."""
    xf = _c(xq, np.int8).astype(np.float64)
    q = _c(q, np.int8)
    M, N = xf.shape[0], q.shape[0]
    acc = np.empty((M, N), np.int32)
    for n0 in range(0, N, _CHANNEL_SLICE):
        n1 = min(N, n0 + _CHANNEL_SLICE)
        acc[:, n0:n1] = _exact_int_matmul(xf, q[n0:n1].astype(np.float64))
    return acc


def forward_w8(x_bits, w_bits):
    """The W8A8 path on the host: quantize both sides, contract, rescale."""
    xq, s_x, rowsum = quantize_act(x_bits)
    s_c, q = quantize_weights_w8(w_bits)
    acc = gemm_w8(xq, q)
    y = epilogue(acc, s_x, s_c)
    return {"xq": xq, "s_x": s_x, "acc": acc, "y": y, "s_c": s_c, "q": q}


# --- W4A16 sibling: FP16 activations, the same 4-bit weights (reading R14) --

def gemm_w4a16(mode, x_bits, s_c, q, s_g, z):
    """(y, absum) float64 [M,N]: y = X . W^T with W^ = s_c * s_g * (q - z)
    (per-channel: s_c * (q - z)); absum = s_c * sum_k |X * W8^|."""
    x = _c(x_bits, np.uint16)
    q = _c(q, np.uint8)
    M, K = x.shape
    N = q.shape[0]
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    sg = None if s_g is None else _c(s_g, np.uint8)
    _check(_load().orc_gemm_w4a16(mode, _p(x), _p(_c(s_c, np.uint16)), _p(q), _p(sg),
                                  _p(_c(z, np.uint8)), M, N, K, _p(y), _p(a)), "gemm_w4a16")
    return y, a


def gemm_w4a16_points(mode, x_bits, s_c, q, s_g, z, ms, ns):
    x = _c(x_bits, np.uint16)
    q = _c(q, np.uint8)
    M, K = x.shape
    N = q.shape[0]
    ms = _c(np.asarray(ms, np.int64), np.int64)
    ns = _c(np.asarray(ns, np.int64), np.int64)
    y = np.empty(len(ms), np.float64)
    a = np.empty(len(ms), np.float64)
    sg = None if s_g is None else _c(s_g, np.uint8)
    _check(_load().orc_gemm_w4a16_points(mode, _p(x), _p(_c(s_c, np.uint16)), _p(q), _p(sg),
                                         _p(_c(z, np.uint8)), M, N, K, len(ms), _p(ms), _p(ns),
                                         _p(y), _p(a)), "gemm_w4a16_points")
    return y, a


def gemm_w4a16_matmul(mode, x_bits, s_c, q, s_g, z):
    """(y, absum) of gemm_w4a16() as library matrix products in float64: y =
    (X . W8^T) * s_c[n] and absum = (|X| . |W8|^T) * s_c[n], with X the exact
    FP16 values and W8 the integer weights of weights_int(). The float64 sums
    are not exact here (X is not integral); their rounding, at most about
    K * 2^-53 * absum, is many orders below any FP32 accumulation bound."""
    x = f16_bits_to_f64(_c(x_bits, np.uint16)).reshape(np.shape(x_bits))
    xa = np.abs(x)
    q = _c(q, np.uint8)
    sc = f16_bits_to_f64(_c(s_c, np.uint16))
    M, N = x.shape[0], q.shape[0]
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    for n0 in range(0, N, _CHANNEL_SLICE):
        n1 = min(N, n0 + _CHANNEL_SLICE)
        sg = None if s_g is None else np.asarray(s_g)[n0:n1]
        w = weights_int(mode, q[n0:n1], sg, np.asarray(z)[n0:n1]).astype(np.float64)
        y[:, n0:n1] = (x @ w.T) * sc[None, n0:n1]
        a[:, n0:n1] = (xa @ np.abs(w).T) * sc[None, n0:n1]
    return y, a


def forward_w4a16(mode, x_bits, w_bits):
    """The W4A16 path on the host: quantize the weights (QoQ, either mode), contract
    the FP16 activations with the dequantized weights."""
    wq = quantize_weights(mode, w_bits)
    y, absum = gemm_w4a16(mode, x_bits, wq["s_c"], wq["q"], wq["s_g"], wq["z"])
    return {"y": y, "absum": absum, **wq}


# --- Fused producer of the down projection's input (reading R15) -----------

def exp_f32(values) -> np.ndarray:
    """The oracle's fp32 exponential (Cody-Waite reduction + degree-7 Taylor)."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32).ravel())
    out = np.empty(v.size, np.float32)
    _load().orc_exp_f32_array(_p(v), v.size, _p(out))
    return out


def silu_mul(gate_up_bits):
    """gate_up [M, 2I] FP16 bits -> h [M, I] FP16 bits, h = f16(SiLU(gate) * up)."""
    gu = _c(gate_up_bits, np.uint16)
    M, I2 = gu.shape
    if I2 % 2:
        raise ValueError("gate_up must have an even number of columns")
    h = np.empty((M, I2 // 2), np.uint16)
    _check(_load().orc_silu_mul(_p(gu), M, I2 // 2, _p(h)), "silu_mul")
    return h


def silu_mul_quantize_act(gate_up_bits):
    """The fused producer: (h, xq, s_x, rowsum) with h = f16(SiLU(gate) * up)
    and (xq, s_x, rowsum) = quantize_act(h)."""
    h = silu_mul(gate_up_bits)
    xq, s_x, rowsum = quantize_act(h)
    return h, xq, s_x, rowsum


# --- RMSNorm producer (reading R17) -------------------------------------------

def rmsnorm(x_bits, gamma_bits, eps, want_r=False):
    """x [M, K] FP16 bits, gamma [K] FP16 bits, eps > 0 -> y [M, K] FP16 bits
    (and r [M] float32 when want_r)."""
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    y = np.empty((M, K), np.uint16)
    r = np.empty((M,), np.float32)
    _check(_load().orc_rmsnorm(_p(x), _p(_c(gamma_bits, np.uint16)), eps, M, K, _p(y), _p(r)),
           "rmsnorm")
    return (y, r) if want_r else y


def rmsnorm_quantize_act(x_bits, gamma_bits, eps):
    """The fused producer: (y, xq, s_x, rowsum) with y = rmsnorm(x) and
    (xq, s_x, rowsum) = quantize_act(y)."""
    y = rmsnorm(x_bits, gamma_bits, eps)
    xq, s_x, rowsum = quantize_act(y)
    return y, xq, s_x, rowsum


# --- KV4 decode attention with SmoothAttention (reading R16) ---------------

def kv4_smooth_scales(k_bits):
    """Calibration keys [T, H, d] FP16 bits -> lambda [H, d] FP16 bits."""
    k = _c(k_bits, np.uint16)
    T, H, d = k.shape
    lam = np.empty((H, d), np.uint16)
    _check(_load().orc_kv4_smooth_scales(_p(k), T, H, d, _p(lam)), "kv4_smooth_scales")
    return lam


def kv4_quantize(k_bits, v_bits, lambda_bits, Tcap=None):
    """Keys and values [B, T, H, d] FP16 bits -> cache dict: kq, vq uint8 [B, H, Tcap, d]
    (one code per byte), ks, vs FP16 bits [B, H, Tcap], kz, vz uint8 [B, H, Tcap]."""
    k = _c(k_bits, np.uint16)
    v = _c(v_bits, np.uint16)
    B, T, H, d = k.shape
    Tcap = T if Tcap is None else Tcap
    out = {"kq": np.zeros((B, H, Tcap, d), np.uint8), "vq": np.zeros((B, H, Tcap, d), np.uint8),
           "ks": np.zeros((B, H, Tcap), np.uint16), "vs": np.zeros((B, H, Tcap), np.uint16),
           "kz": np.zeros((B, H, Tcap), np.uint8), "vz": np.zeros((B, H, Tcap), np.uint8)}
    _check(_load().orc_kv4_quantize(_p(k), _p(v), _p(_c(lambda_bits, np.uint16)), B, T, H, d, Tcap,
                                    _p(out["kq"]), _p(out["ks"]), _p(out["kz"]), _p(out["vq"]),
                                    _p(out["vs"]), _p(out["vz"])), "kv4_quantize")
    return out


def kv4_decode_attention(q_bits, lambda_bits, cache, lens):
    """q [B, Hq, d] FP16 bits, lambda [H, d], the cache of kv4_quantize, lens int32 [B]
    -> o float64 [B, Hq, d]."""
    q = _c(q_bits, np.uint16)
    B, Hq, d = q.shape
    H = cache["kq"].shape[1]
    Tcap = cache["kq"].shape[2]
    lens = _c(np.asarray(lens, np.int32), np.int32)
    o = np.empty((B, Hq, d), np.float64)
    c = {k: np.ascontiguousarray(v) for k, v in cache.items()}
    _check(_load().orc_kv4_decode_attention(_p(q), _p(_c(lambda_bits, np.uint16)), _p(c["kq"]),
                                            _p(c["ks"]), _p(c["kz"]), _p(c["vq"]), _p(c["vs"]),
                                            _p(c["vz"]), _p(lens), B, Hq, H, d, Tcap, _p(o)),
           "kv4_decode_attention")
    return o
