"""Helpers shared by the GPU parity tests: move arrays between numpy (the
oracle's side) and torch device tensors (the library's side)."""
import numpy as np
import torch

import oracle

DEV = "cuda:0"


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def f16_dev(bits: np.ndarray) -> torch.Tensor:
    return to_dev(bits.astype(np.uint16), torch.float16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def assert_y_close(y_gpu_bits: np.ndarray, y_ref: np.ndarray, what: str = ""):
    """FP16 output within 1e-3 * max|Y| of the oracle's exact value, and within
    one FP16 rounding (plus fp32 rounding) of it element by element."""
    yg = y_gpu_bits.view(np.float16).astype(np.float64)
    ref = np.asarray(y_ref, np.float64)
    # Exact values at or beyond 65520 round to +-inf in FP16 (round to nearest even).
    over = np.abs(ref) >= 65520.0
    assert np.all(np.isinf(yg[over]) & (np.sign(yg[over]) == np.sign(ref[over]))), what
    yg, ref = yg[~over], ref[~over]
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = np.abs(yg - ref)
    assert err.max(initial=0.0) <= 1e-3 * scale + 1e-30, (what, err.max(), scale)
    # Each output is f16(fp32 product): at most one FP16 ulp from the exact value
    # (half an ulp for the final rounding, plus fp32 rounding of the product).
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    ulp = np.maximum(ulp, 2.0**-24)
    assert np.all(err <= ulp), (what, float((err / ulp).max()))


def quantize_all(mode, x_bits, w_bits):
    """The oracle's view of one layer: activations, weights and the blob."""
    xq, s_x, rowsum = oracle.quantize_act(x_bits)
    wq = oracle.quantize_weights(mode, w_bits)
    blob = oracle.pack(mode, wq["q"], wq["s_g"], wq["z"])
    return xq, s_x, rowsum, wq, blob
