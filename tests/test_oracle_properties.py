"""Pin the oracle to what the pages and the mathematics fix, beyond the
hand-worked fixtures: exhaustive sweeps, error bounds, brute force on tiny
inputs, a library contraction, special cases and the end-to-end approximation
of the real product.

Each check targets a plausible mistake: a wrong rounding mode or FP16 encoding
(fp16 sweep), a floor instead of a ceiling or a sign error in the group zero
(exhaustive stage-2 sweep), a dropped clip or a wrong range constant (headroom
and stage-1 bounds), a transposed operand or a wrong scale (brute force,
library matmul, end-to-end product).
"""
import numpy as np
import pytest

import oracle
from quantized_gemm_qoq_amd import workloads

G128 = oracle.MODE_G128
PC = oracle.MODE_PER_CHANNEL


# ---------------------------------------------------------------- fp16 -----
def test_f32_to_f16_matches_numpy_exhaustive_fp16_grid():
    """Every binary16 value, every midpoint between neighbours (ties) and the
    floats just either side of each midpoint round as numpy's RNE cast does."""
    bits = np.arange(0, 0x7C00, dtype=np.uint32)  # all finite non-negative
    vals = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    nxt = (bits + 1).astype(np.uint16).view(np.float16).astype(np.float32)
    mids = ((vals.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    cases = np.concatenate([vals, mids, up, dn])
    cases = np.concatenate([cases, -cases])
    with np.errstate(over="ignore"):
        want = cases.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_f16_bits(cases), want)


def test_f32_to_f16_matches_numpy_random_bits():
    rng = np.random.default_rng(7)
    b = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = b.view(np.float32)
    f = f[np.isfinite(f)]
    with np.errstate(over="ignore"):
        want = f.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_f16_bits(f), want)


def test_f16_decode_matches_numpy():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7C00) != 0x7C00
    got = oracle.f16_bits_to_f64(bits[finite])
    np.testing.assert_array_equal(got, bits[finite].view(np.float16).astype(np.float64))


# -------------------------------------------------------------- stage 2 ----
def _stage2_sweep_rows():
    """Rows whose groups realise every (mn, mx) with -119 <= mn <= 0 <= mx <= 119
    and every integer w8 in [mn, mx]. Group 0 of each row holds +-119 so that
    s_c = 2^-8 exactly and stage 1 is the identity on the integers."""
    groups, meta = [], []
    for mn in range(-119, 1):
        for mx in range(0, 120):
            vals = list(range(mn, mx + 1))
            # 126 free slots per group besides mn and mx
            for start in range(0, len(vals), 126):
                chunk = vals[start:start + 126]
                grp = np.zeros(128, np.int64)
                grp[0], grp[1] = mn, mx
                grp[2:2 + len(chunk)] = chunk
                grp[2 + len(chunk):] = chunk[-1]
                groups.append(grp)
                meta.append((mn, mx))
    per_row = 32
    nrows = (len(groups) + per_row - 1) // per_row
    anchor = np.zeros(128, np.int64)
    anchor[0], anchor[1] = 119, -119
    w8 = np.zeros((nrows, 128 * (per_row + 1)), np.int64)
    for r in range(nrows):
        w8[r, :128] = anchor
    for i, grp in enumerate(groups):
        r, c = divmod(i, per_row)
        w8[r, 128 * (c + 1):128 * (c + 2)] = grp
    # rows padded with zero groups: those groups are (0, 0)
    return w8, meta, per_row


def test_stage2_exhaustive_headroom_and_error_bound():
    w8, meta, per_row = _stage2_sweep_rows()
    w = (w8.astype(np.float64) * 2.0**-8).astype(np.float16)
    assert np.array_equal(w.astype(np.float64), w8 * 2.0**-8)
    out = oracle.quantize_weights(G128, w.view(np.uint16), want_w8=True)
    assert np.all(out["s_c"] == 0x1C00)  # 2^-8
    np.testing.assert_array_equal(out["w8"].astype(np.int64), w8)

    q = out["q"].astype(np.int64)
    s_g = out["s_g"].astype(np.int64)
    z = out["z"].astype(np.int64)
    N, K = q.shape
    G = K // 128
    sg_full = np.repeat(s_g, 128, axis=1)
    z_full = np.repeat(z, 128, axis=1)
    w8hat = (q - z_full) * sg_full

    # Codes and zero in UINT4, integer scale in [1, 16].
    assert q.min() >= 0 and q.max() <= 15
    assert z.min() >= 0 and z.max() <= 15
    assert s_g.min() >= 1 and s_g.max() <= 16
    # The protective range keeps the unpacked INT8 value inside INT8: the pages'
    # claim. The tight range is [-121, 121].
    assert w8hat.min() >= -128 and w8hat.max() <= 127
    assert w8hat.min() == -121 and w8hat.max() == 121
    # Stage-2 error: the clip never binds, so every value is within s_g/2.
    assert np.all(2 * np.abs(w8hat - w8) <= sg_full)

    # The group scale is the smallest integer that covers the range in 15 steps:
    # 15*s_g >= mx - mn and 15*(s_g - 1) < mx - mn (unless s_g = 1).
    mn = np.minimum(0, w8.reshape(N, G, 128).min(axis=2))
    mx = np.maximum(0, w8.reshape(N, G, 128).max(axis=2))
    rng = mx - mn
    assert np.all(15 * s_g >= rng)
    assert np.all((s_g == 1) | (15 * (s_g - 1) < rng))
    # The zero maps mn onto the code grid: |z*s_g + mn| <= s_g/2.
    assert np.all(2 * np.abs(z * s_g + mn) <= s_g)

    # Every (mn, mx) pair was realised.
    seen = set(zip(mn[:, 1:].ravel().tolist(), mx[:, 1:].ravel().tolist()))
    assert set(meta) <= seen


def test_headroom_119_is_tight():
    """With a protective range of 120 instead of 119 the same stage-2 formulas
    overflow INT8: mn = -119, mx = 120, w8 = 120 gives s_g = 16, z = 7,
    q = round(7.5) + 7 = 15 and (q - z) * s_g = 128 (pure arithmetic of the
    stage-2 equation, independent of the oracle)."""
    mn, mx, w = -119, 120, 120
    sg = -(-(mx - mn) // 15)
    z = round(-mn / sg)
    qv = min(15, max(0, round(w / sg) + z))
    assert (sg, z, qv) == (16, 7, 15)
    assert (qv - z) * sg == 128


# -------------------------------------------------------------- stage 1 ----
@pytest.mark.parametrize("seed", [1, 2])
def test_stage1_bounds_random(seed):
    w = workloads.random_fp16((64, 1024), seed, 0.02)
    w[3, 5] = 0.0
    w[7] = 0.0  # an all-zero row
    w[9, :] = 0.25  # a constant row
    wb = w.numpy().view(np.uint16)
    out = oracle.quantize_weights(G128, wb, want_w8=True)
    wf = w.numpy().astype(np.float64)
    s_c = oracle.f16_bits_to_f64(out["s_c"])
    amax = np.abs(wf).max(axis=1)
    # s_c is max|W|/119 rounded to FP16: within half an FP16 ulp (2^-11 relative).
    nz = amax > 0
    assert np.all(np.abs(s_c[nz] - amax[nz] / 119) <= (amax[nz] / 119) * 2.0**-11)
    assert s_c[7] == 0 and np.all(out["q"][7] == 0) and np.all(out["z"][7] == 0)
    w8 = out["w8"].astype(np.float64)
    assert np.abs(w8).max() <= 119
    ratio = wf[nz] / s_c[nz, None]
    # Round to nearest: within 1/2 (plus the fp32 division's rounding), no clip binds.
    assert np.all(np.abs(w8[nz] - ratio) <= 0.5 + 1e-4)
    # The largest magnitude of each row maps to +-119.
    arg = np.abs(wf).argmax(axis=1)
    assert np.all(np.abs(w8[np.arange(64)[nz], arg[nz]]) == 119)
    # A constant row: every element is the row max.
    assert np.all(w8[9] == 119)


def test_reconstruction_bound_g128_and_per_channel():
    x16 = workloads.random_fp16((48, 1024), 11, 0.02)
    x16[5, 100] = 0.9  # an outlier in one row
    wb = x16.numpy().view(np.uint16)
    wf = x16.numpy().astype(np.float64)
    out = oracle.quantize_weights(G128, wb)
    what = oracle.dequantize_weights(G128, out["s_c"], out["q"], out["s_g"], out["z"])
    s_c = oracle.f16_bits_to_f64(out["s_c"])[:, None]
    sg = np.repeat(out["s_g"].astype(np.float64), 128, axis=1)
    # |W^ - W| <= s_c * (1/2 + s_g/2): stage-1 rounding plus stage-2 rounding.
    assert np.all(np.abs(what - wf) <= s_c * (0.5 + 1e-4 + sg / 2))
    rel_g = np.linalg.norm(what - wf) / np.linalg.norm(wf)

    pc = oracle.quantize_weights(PC, wb)
    what_pc = oracle.dequantize_weights(PC, pc["s_c"], pc["q"], None, pc["z"])
    s_pc = oracle.f16_bits_to_f64(pc["s_c"])[:, None]
    assert np.all(np.abs(what_pc - wf) <= s_pc * 0.51)
    rel_pc = np.linalg.norm(what_pc - wf) / np.linalg.norm(wf)
    # Group quantization is finer than one range per row.
    assert rel_g < rel_pc < 0.5


# ----------------------------------------------------------- activations ---
def test_act_quant_bounds_random():
    x = workloads.random_fp16((40, 2048), 5, 1.0)
    x[0] = 0.0
    x[1, 7] = -30.0
    x[2, :] = -1.5
    xb = x.numpy().view(np.uint16)
    xq, s_x, rowsum = oracle.quantize_act(xb)
    xf = x.numpy().astype(np.float64)
    s = oracle.f16_bits_to_f64(s_x)
    assert s[0] == 0 and np.all(xq[0] == 0) and rowsum[0] == 0
    nz = s > 0
    err = np.abs(xq[nz].astype(np.float64) * s[nz, None] - xf[nz])
    assert np.all(err <= s[nz, None] * (0.5 + 1e-4))
    assert np.abs(xq.astype(np.int64)).max() <= 127
    arg = np.abs(xf).argmax(axis=1)
    assert np.all(np.abs(xq[np.arange(40)[nz], arg[nz]]) == 127)
    assert xq[1, 7] == -127
    assert np.all(xq[2] == -127)
    np.testing.assert_array_equal(rowsum, xq.astype(np.int64).sum(axis=1))


def test_act_scale_underflow_gives_zero_codes():
    # max|X| = 2^-24 (the smallest FP16 subnormal): max/127 rounds to 0 in FP16.
    x = np.zeros((1, 128), np.uint16)
    x[0, 3] = 0x0001
    xq, s_x, rowsum = oracle.quantize_act(x)
    assert s_x[0] == 0 and np.all(xq == 0) and rowsum[0] == 0


# ------------------------------------------------------------------ GEMM ---
def _brute(mode, xq, q, s_g, z):
    M, K = xq.shape
    N = q.shape[0]
    acc = np.zeros((M, N), np.int64)
    for m in range(M):
        for n in range(N):
            s = 0
            for k in range(K):
                if mode == G128:
                    wv = (int(q[n, k]) - int(z[n, k // 128])) * int(s_g[n, k // 128])
                else:
                    wv = int(q[n, k]) - int(z[n])
                s += int(xq[m, k]) * wv
            acc[m, n] = s
    return acc


@pytest.mark.parametrize("mode", [G128, PC])
@pytest.mark.parametrize("shape", [(1, 128, 3), (5, 256, 7), (16, 512, 16)])
def test_gemm_brute_force_tiny(mode, shape):
    M, K, N = shape
    x = workloads.random_fp16((M, K), 100 + K, 1.0).numpy().view(np.uint16)
    w = workloads.random_fp16((N, K), 200 + K, 0.02).numpy().view(np.uint16)
    xq, s_x, rowsum = oracle.quantize_act(x)
    wq = oracle.quantize_weights(mode, w)
    acc = oracle.gemm(mode, xq, wq["q"], wq["s_g"], wq["z"])
    np.testing.assert_array_equal(acc, _brute(mode, xq, wq["q"], wq["s_g"], wq["z"]))
    ms = np.repeat(np.arange(M), N)
    ns = np.tile(np.arange(N), M)
    pts = oracle.gemm_points(mode, xq, wq["q"], wq["s_g"], wq["z"], ms, ns)
    np.testing.assert_array_equal(pts, acc.ravel())


@pytest.mark.parametrize("mode", [G128, PC])
def test_gemm_matches_library_matmul(mode):
    M, K, N = 37, 1024, 96
    x = workloads.random_fp16((M, K), 31, 1.0).numpy().view(np.uint16)
    w = workloads.random_fp16((N, K), 32, 0.02).numpy().view(np.uint16)
    xq, s_x, rowsum = oracle.quantize_act(x)
    wq = oracle.quantize_weights(mode, w)
    q = wq["q"].astype(np.int64)
    if mode == G128:
        w8 = (q - np.repeat(wq["z"], 128, 1)) * np.repeat(wq["s_g"], 128, 1)
    else:
        w8 = q - wq["z"].astype(np.int64)[:, None]
    want = np.matmul(xq.astype(np.int64), w8.T)
    acc = oracle.gemm(mode, xq, wq["q"], wq["s_g"], wq["z"])
    np.testing.assert_array_equal(acc, want)
    if mode == PC:
        # The epilogue form the GPU uses: sum xq*q - z*rowsum.
        factored = np.matmul(xq.astype(np.int64), q.T) - np.outer(rowsum, wq["z"].astype(np.int64))
        np.testing.assert_array_equal(acc, factored)


MATMUL_SHAPES = [(1, 16, 128), (7, 48, 384), (33, 272, 1024), (130, 2064, 256), (3, 16, 132096)]


@pytest.mark.parametrize("mode", [G128, PC])
@pytest.mark.parametrize("M,N,K", MATMUL_SHAPES)
def test_gemm_matmul_equals_the_c_loops(mode, M, N, K):
    """The library-product form of the accumulator (used on full-size layers)
    equals the C oracle's int64 loops element by element, on ragged shapes
    (M != N, a channel count past one slice of the product) and at the largest
    K; activations include the extreme codes -128 and 127."""
    x = workloads.random_fp16((M, K), 600 + M, 1.0).numpy().view(np.uint16)
    w = workloads.random_fp16((N, K), 700 + N, 0.02).numpy().view(np.uint16)
    xq, _, _ = oracle.quantize_act(x)
    xq = xq.copy()
    xq[0, :3] = [-128, 127, -127]
    wq = oracle.quantize_weights(mode, w)
    want = oracle.gemm(mode, xq, wq["q"], wq["s_g"], wq["z"])
    np.testing.assert_array_equal(oracle.gemm_matmul(mode, xq, wq["q"], wq["s_g"], wq["z"]), want)


def test_gemm_matmul_refuses_int32_overflow():
    K = 132096
    xq = np.full((1, K), -128, np.int8)
    q = np.zeros((16, K), np.uint8)
    s_g = np.full((16, K // 128), 16, np.uint8)
    z = np.full((16, K // 128), 8, np.uint8)
    with pytest.raises(OverflowError):
        oracle.gemm_matmul(G128, xq, q, s_g, z)


@pytest.mark.parametrize("M,N,K", MATMUL_SHAPES[:4])
def test_gemm_w8_matmul_equals_the_c_loops(M, N, K):
    x = workloads.random_fp16((M, K), 800 + M, 1.0).numpy().view(np.uint16)
    w = workloads.random_fp16((N, K), 900 + N, 0.02).numpy().view(np.uint16)
    xq, _, _ = oracle.quantize_act(x)
    _, q = oracle.quantize_weights_w8(w)
    np.testing.assert_array_equal(oracle.gemm_w8_matmul(xq, q), oracle.gemm_w8(xq, q))


@pytest.mark.parametrize("mode", [G128, PC])
@pytest.mark.parametrize("M,N,K", MATMUL_SHAPES[:4])
def test_gemm_w4a16_matmul_matches_the_c_loops(mode, M, N, K):
    """Both forms sum in fp64 in different orders: they agree far inside the
    rounding of a float64 sum (K * 2^-52 of the absolute sum)."""
    x = workloads.random_fp16((M, K), 1000 + M, 1.0).numpy().view(np.uint16)
    w = workloads.random_fp16((N, K), 1100 + N, 0.02).numpy().view(np.uint16)
    wq = oracle.quantize_weights(mode, w)
    y0, a0 = oracle.gemm_w4a16(mode, x, wq["s_c"], wq["q"], wq["s_g"], wq["z"])
    y1, a1 = oracle.gemm_w4a16_matmul(mode, x, wq["s_c"], wq["q"], wq["s_g"], wq["z"])
    tol = K * 2.0**-52 * a0
    assert np.all(np.abs(y1 - y0) <= tol)
    assert np.all(np.abs(a1 - a0) <= tol)


def test_epilogue_points_equals_epilogue_everywhere():
    """orc_epilogue_points, at every (m, n) of a non-square shape in shuffled
    order, equals orc_epilogue; the scales are distinct per row and per channel
    (and the two vectors have different lengths), so a swapped or transposed
    index fails."""
    M, N = 37, 80
    rng = np.random.default_rng(77)
    acc = rng.integers(-(2**31), 2**31, size=(M, N), dtype=np.int64).astype(np.int32)
    s_x = rng.permutation(np.arange(M, dtype=np.uint16) * 7 + 0x3000)  # distinct FP16 scales
    s_c = rng.permutation(np.arange(N, dtype=np.uint16) * 3 + 0x1000)
    y = oracle.epilogue(acc, s_x, s_c)
    order = rng.permutation(M * N)
    ms, ns = order // N, order % N
    yp = oracle.epilogue_points(acc[ms, ns], s_x, s_c, ms, ns)
    np.testing.assert_array_equal(yp, y[ms, ns])
    # and against the definition at a few points, in exact arithmetic
    sx, sc = oracle.f16_bits_to_f64(s_x), oracle.f16_bits_to_f64(s_c)
    for p in range(0, M * N, 97):
        assert yp[p] == float(acc[ms[p], ns[p]]) * sx[ms[p]] * sc[ns[p]]


def test_gemm_int32_range_at_max_k():
    """At K = 132096 the largest reachable products stay inside INT32, and the
    oracle refuses a sum that would not (|xq| = 128 with |W8^| = 128 is outside
    what the quantizers emit)."""
    K = 132096
    xq = np.full((1, K), -127, np.int8)
    q = np.zeros((16, K), np.uint8)
    s_g = np.full((16, K // 128), 11, np.uint8)
    z = np.full((16, K // 128), 11, np.uint8)  # (0 - 11) * 11 = -121, the tight extreme
    acc = oracle.gemm(G128, xq, q, s_g, z)
    assert np.all(acc == K * 127 * 121)
    xq[:] = -128
    s_g[:] = 16
    z[:] = 8  # (0 - 8) * 16 = -128: K * 128 * 128 > 2^31 - 1
    with pytest.raises(RuntimeError):
        oracle.gemm(G128, xq, q, s_g, z)


def test_epilogue_is_exact_product():
    acc = np.array([[2**30 + 1, -(2**30) - 3]], np.int32)
    s_x = np.array([0x3BFF], np.uint16)  # 1 - 2^-11
    s_c = np.array([0x3BFF, 0x0001], np.uint16)
    y = oracle.epilogue(acc, s_x, s_c)
    a = 1 - 2.0**-11
    assert y[0, 0] == (2**30 + 1) * a * a  # exactly representable in fp64
    assert y[0, 1] == -(2**30 + 3) * a * 2.0**-24


@pytest.mark.parametrize("mode", [G128, PC])
def test_end_to_end_approximates_real_product(mode):
    """Y approximates X W^T: a transposed operand, a missing scale or a wrong
    sign would not."""
    layer = workloads.WORKLOADS["tiny"].layers[0]
    x16, w16 = workloads.generate(layer)
    res = oracle.forward(mode, x16.numpy().view(np.uint16), w16.numpy().view(np.uint16))
    ref = x16.numpy().astype(np.float64) @ w16.numpy().astype(np.float64).T
    rel = np.linalg.norm(res["y"] - ref) / np.linalg.norm(ref)
    assert rel < 0.15, rel
    cos = (res["y"] * ref).sum() / np.linalg.norm(res["y"]) / np.linalg.norm(ref)
    assert cos > 0.99


def test_zero_inputs_give_zero_output():
    x = np.zeros((3, 256), np.uint16)
    w = workloads.random_fp16((16, 256), 3, 0.02).numpy().view(np.uint16)
    for mode in (G128, PC):
        res = oracle.forward(mode, x, w)
        assert np.all(res["y"] == 0) and np.all(res["acc"] == 0)
        res = oracle.forward(mode, w[:2], np.zeros((16, 256), np.uint16))
        assert np.all(res["y"] == 0)


# --------------------------------------------------------- W8A8 sibling ----
def test_w8_quant_bounds_random():
    """Per-channel symmetric INT8: scale within half an FP16 ulp of max|W|/127,
    codes within 1/2 of W/s_c, the row maximum at +-127, zero rows zero."""
    w = workloads.random_fp16((64, 1024), 21, 0.02)
    w[7] = 0.0
    w[9, :] = -0.25
    w[11, 3] = 0.7  # an outlier
    wb = w.numpy().view(np.uint16)
    s_c_bits, q = oracle.quantize_weights_w8(wb)
    wf = w.numpy().astype(np.float64)
    s_c = oracle.f16_bits_to_f64(s_c_bits)
    amax = np.abs(wf).max(axis=1)
    nz = amax > 0
    assert np.all(np.abs(s_c[nz] - amax[nz] / 127) <= (amax[nz] / 127) * 2.0**-11)
    assert s_c[7] == 0 and not q[7].any()
    qf = q.astype(np.float64)
    assert np.abs(qf).max() <= 127
    assert np.all(np.abs(qf[nz] - wf[nz] / s_c[nz, None]) <= 0.5 + 1e-4)
    arg = np.abs(wf).argmax(axis=1)
    assert np.all(np.abs(qf[np.arange(64)[nz], arg[nz]]) == 127)
    assert np.all(q[9] == -127)
    # W8 is much finer than W4 per channel.
    rel8 = np.linalg.norm(qf * s_c[:, None] - wf) / np.linalg.norm(wf)
    pc = oracle.quantize_weights(PC, wb)
    what_pc = oracle.dequantize_weights(PC, pc["s_c"], pc["q"], None, pc["z"])
    rel4 = np.linalg.norm(what_pc - wf) / np.linalg.norm(wf)
    assert rel8 < rel4 / 8


def test_w8_pack_is_the_tile_permutation():
    """The packed INT8 blob read back through a plain reshape of the written
    layout (tile t, group g, k-step s, lane block j, channel c, byte i)
    returns every code."""
    N, K = 48, 384
    rng = np.random.default_rng(3)
    q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    blob = oracle.pack_w8(q).view(np.int8)
    T, G = N // 16, K // 128
    v = blob.reshape(T, G, 2, 4, 16, 16)  # [t, g, s, j, c, i]
    back = v.transpose(0, 4, 1, 2, 3, 5).reshape(N, K)  # n = 16t + c, k = 128g + 64s + 16j + i
    np.testing.assert_array_equal(back, q)


@pytest.mark.parametrize("shape", [(1, 128, 3), (6, 256, 16)])
def test_w8_gemm_brute_force_tiny(shape):
    M, K, N = shape
    x = workloads.random_fp16((M, K), 300 + K, 1.0).numpy().view(np.uint16)
    w = workloads.random_fp16((N, K), 400 + K, 0.02).numpy().view(np.uint16)
    xq, _, _ = oracle.quantize_act(x)
    _, q = oracle.quantize_weights_w8(w)
    want = np.zeros((M, N), np.int64)
    for m in range(M):
        for n in range(N):
            want[m, n] = sum(int(xq[m, k]) * int(q[n, k]) for k in range(K))
    acc = oracle.gemm_w8(xq, q)
    np.testing.assert_array_equal(acc, want)
    ms = np.repeat(np.arange(M), N)
    ns = np.tile(np.arange(N), M)
    np.testing.assert_array_equal(oracle.gemm_w8_points(xq, q, ms, ns), acc.ravel())


def test_w8_gemm_matches_library_matmul_and_range():
    M, K, N = 29, 2048, 80
    x = workloads.random_fp16((M, K), 41, 1.0).numpy().view(np.uint16)
    w = workloads.random_fp16((N, K), 42, 0.02).numpy().view(np.uint16)
    xq, _, _ = oracle.quantize_act(x)
    _, q = oracle.quantize_weights_w8(w)
    want = np.matmul(xq.astype(np.int64), q.astype(np.int64).T)
    np.testing.assert_array_equal(oracle.gemm_w8(xq, q), want)
    # At the largest K the extreme codes stay inside INT32 (127 * 127 * 132096).
    Kmax = 132096
    xa = np.full((1, Kmax), -127, np.int8)
    qa = np.full((16, Kmax), 127, np.int8)
    assert np.all(oracle.gemm_w8(xa, qa) == -127 * 127 * Kmax)
    with pytest.raises(RuntimeError):
        oracle.gemm_w8(np.full((1, Kmax), -128, np.int8), np.full((16, Kmax), -128, np.int8))


def test_w8_end_to_end_approximates_real_product():
    layer = workloads.WORKLOADS["tiny"].layers[0]
    x16, w16 = workloads.generate(layer)
    res = oracle.forward_w8(x16.numpy().view(np.uint16), w16.numpy().view(np.uint16))
    ref = x16.numpy().astype(np.float64) @ w16.numpy().astype(np.float64).T
    rel = np.linalg.norm(res["y"] - ref) / np.linalg.norm(ref)
    assert rel < 0.03, rel
    w4 = oracle.forward(G128, x16.numpy().view(np.uint16), w16.numpy().view(np.uint16))
    rel4 = np.linalg.norm(w4["y"] - ref) / np.linalg.norm(ref)
    assert rel < rel4


# -------------------------------------------------------- W4A16 sibling ----
def test_w4a16_matches_exact_rational_sum():
    """The fp64 contraction against exact rational arithmetic (Python
    fractions) on a small case spanning two groups and both modes."""
    from fractions import Fraction
    M, K, N = 3, 256, 16
    x = workloads.random_fp16((M, K), 51, 1.0).numpy()
    x[0, 5] = np.float16(6e-8)  # a subnormal activation
    w = workloads.random_fp16((N, K), 52, 0.02).numpy().view(np.uint16)
    for mode in (G128, PC):
        wq = oracle.quantize_weights(mode, w)
        y, absum = oracle.gemm_w4a16(mode, x.view(np.uint16), wq["s_c"], wq["q"], wq["s_g"],
                                     wq["z"])
        sc = oracle.f16_bits_to_f64(wq["s_c"])
        for m in range(M):
            for n in range(N):
                tot = Fraction(0)
                for k in range(K):
                    if mode == G128:
                        wv = (int(wq["q"][n, k]) - int(wq["z"][n, k // 128])) * int(wq["s_g"][n, k // 128])
                    else:
                        wv = int(wq["q"][n, k]) - int(wq["z"][n])
                    tot += Fraction(float(x[m, k])) * wv
                exact = tot * Fraction(float(sc[n]))
                assert abs(Fraction(y[m, n]) - exact) <= Fraction(2.0**-50) * Fraction(absum[m, n]) + Fraction(2.0**-1074)


def test_w4a16_matches_library_matmul_of_dequantized_weights():
    M, K, N = 19, 1024, 64
    x = workloads.random_fp16((M, K), 53, 1.0).numpy()
    w = workloads.random_fp16((N, K), 54, 0.02).numpy().view(np.uint16)
    for mode in (G128, PC):
        wq = oracle.quantize_weights(mode, w)
        what = oracle.dequantize_weights(mode, wq["s_c"], wq["q"], wq["s_g"], wq["z"])
        want = np.matmul(x.astype(np.float64), what.T)
        y, absum = oracle.gemm_w4a16(mode, x.view(np.uint16), wq["s_c"], wq["q"], wq["s_g"], wq["z"])
        assert np.all(np.abs(y - want) <= 1e-13 * absum)
        ms = np.array([0, M - 1, 7]); ns = np.array([N - 1, 0, 33])
        yp, ap = oracle.gemm_w4a16_points(mode, x.view(np.uint16), wq["s_c"], wq["q"], wq["s_g"],
                                          wq["z"], ms, ns)
        np.testing.assert_array_equal(yp, y[ms, ns])
        np.testing.assert_array_equal(ap, absum[ms, ns])


def test_w4a16_end_to_end_is_closer_than_w4a8():
    """Keeping the activations in FP16 removes the activation rounding: W4A16
    approximates X W^T at least as well as W4A8 on the same weights."""
    layer = workloads.WORKLOADS["tiny"].layers[0]
    x16, w16 = workloads.generate(layer)
    xb, wb = x16.numpy().view(np.uint16), w16.numpy().view(np.uint16)
    ref = x16.numpy().astype(np.float64) @ w16.numpy().astype(np.float64).T
    a16 = oracle.forward_w4a16(G128, xb, wb)
    a8 = oracle.forward(G128, xb, wb)
    r16 = np.linalg.norm(a16["y"] - ref) / np.linalg.norm(ref)
    r8 = np.linalg.norm(a8["y"] - ref) / np.linalg.norm(ref)
    assert r16 <= r8 < 0.15


# --------------------------------------------------- fused SiLU * up + quant ----
def test_exp_f32_against_libm():
    """The oracle's fp32 exponential is within 1.5 fp32 ulps of the exact
    value over its whole finite range, exact at 0, and follows its cut-offs."""
    x = np.concatenate([np.linspace(-86, 88, 1_000_001), np.linspace(-1, 1, 200_001),
                        np.array([-86.0, 88.0, 1e-30, -1e-30])]).astype(np.float32)
    e = oracle.exp_f32(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(e - ref) <= 1.5 * ulp)
    assert oracle.exp_f32([0.0])[0] == 1.0
    assert np.all(oracle.exp_f32([88.001, 100.0, 65504.0]) == np.inf)
    assert np.all(oracle.exp_f32([-86.001, -100.0, -65504.0]) == 0.0)


def test_silu_mul_matches_fp64_definition():
    """h = f16(SiLU(g) * u) is within one FP16 rounding (plus a few fp32 ulps)
    of the exact product, and equals the FP16 rounding of the fp64 value
    almost everywhere (a difference needs the fp32 value and the fp64 value on
    opposite sides of an FP16 rounding boundary)."""
    M, I = 64, 1024
    g = (workloads.random_fp16((M, I), 61, 3.0)).numpy()
    u = (workloads.random_fp16((M, I), 62, 1.0)).numpy()
    g[0, :8] = [0, 1e-4, -1e-4, 20, -20, 87, -87, 11.0]
    gu = np.concatenate([g, u], axis=1)
    h = oracle.silu_mul(gu.view(np.uint16)).view(np.float16).astype(np.float64)
    gd, ud = g.astype(np.float64), u.astype(np.float64)
    exact = gd / (1.0 + np.exp(-gd)) * ud
    ulp16 = np.spacing(np.abs(exact).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(h - exact) <= 0.5 * ulp16 + 2.0**-20 * np.abs(exact) + 2.0**-25)
    same = h == exact.astype(np.float16).astype(np.float64)
    assert same.mean() > 0.999


def test_silu_mul_quantize_is_the_composition():
    M, I = 5, 384
    gu = workloads.random_fp16((M, 2 * I), 63, 2.0).numpy().view(np.uint16)
    h, xq, s_x, rowsum = oracle.silu_mul_quantize_act(gu)
    xq2, s_x2, rs2 = oracle.quantize_act(oracle.silu_mul(gu))
    np.testing.assert_array_equal(xq, xq2)
    np.testing.assert_array_equal(s_x, s_x2)
    np.testing.assert_array_equal(rowsum, rs2)


# ------------------------------------------- KV4 attention + SmoothAttention ----
def _kv_inputs(B, T, H, d, seed, k_outliers=()):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, T, H, d)).astype(np.float32)
    for ch, f in k_outliers:
        k[..., ch] *= f
    v = rng.standard_normal((B, T, H, d)).astype(np.float32)
    return k.astype(np.float16), v.astype(np.float16)


def _dequant(cache, which):
    q = cache[which + "q"].astype(np.float64)
    s = cache[which + "s"].view(np.float16).astype(np.float64)[..., None]
    z = cache[which + "z"].astype(np.float64)[..., None]
    return s * (q - z)


def test_smooth_scales_definition_and_effect():
    """lambda^2 recovers each channel's largest |K| to FP16 precision, the
    smoothed keys' channel maxima are sqrt of the originals (the outlier
    channel shrinks toward the rest), and q' . k' equals q . k."""
    B, T, H, d = 1, 64, 2, 128
    k, _ = _kv_inputs(B, T, H, d, 5, k_outliers=[(7, 20.0), (40, 12.0)])
    lam = oracle.kv4_smooth_scales(k.reshape(T, H, d).view(np.uint16))
    lf = lam.view(np.float16).astype(np.float64)
    amax = np.abs(k.astype(np.float64)).max(axis=(0, 1))  # [H, d]
    assert np.all(np.abs(lf**2 - amax) <= amax * 2.0**-9)
    ks = k.astype(np.float64) / lf
    smax = np.abs(ks).max(axis=(0, 1))
    assert np.all(np.abs(smax - np.sqrt(amax)) <= np.sqrt(amax) * 2.0**-9)
    spread_before = amax.max(axis=1) / np.median(amax, axis=1)
    spread_after = smax.max(axis=1) / np.median(smax, axis=1)
    assert np.all(spread_after < spread_before / 2)
    q = np.random.default_rng(6).standard_normal((H, d))
    np.testing.assert_allclose(((q * lf)[None, None] * ks).sum(-1),
                               (q[None, None] * k.astype(np.float64)).sum(-1), rtol=1e-12, atol=1e-12)
    zero = np.zeros((3, 1, 128), np.uint16)
    assert np.all(oracle.kv4_smooth_scales(zero) == np.float16(1.0).view(np.uint16))


def test_kv4_quantize_matches_per_channel_w4_rows_and_bounds():
    """Each cached (token, head) vector is quantized like a per-channel W4 row
    (two functions written separately from the same formulas), with codes
    within half a step of the value."""
    B, T, H, d = 2, 9, 3, 128
    k, v = _kv_inputs(B, T, H, d, 7, k_outliers=[(3, 10.0)])
    lam = oracle.kv4_smooth_scales(k.reshape(B * T, H, d).view(np.uint16))
    c = oracle.kv4_quantize(k.view(np.uint16), v.view(np.uint16), lam, Tcap=12)
    vrows = np.transpose(v, (0, 2, 1, 3)).reshape(-1, d)  # [B*H*T, d]
    pc = oracle.quantize_weights(PC, vrows.view(np.uint16))
    np.testing.assert_array_equal(c["vq"][:, :, :T].reshape(-1, d), pc["q"])
    np.testing.assert_array_equal(c["vs"][:, :, :T].reshape(-1), pc["s_c"])
    np.testing.assert_array_equal(c["vz"][:, :, :T].reshape(-1), pc["z"])
    assert not c["kq"][:, :, T:].any() and not c["ks"][:, :, T:].any()  # capacity untouched
    kd = _dequant(c, "k")[:, :, :T]
    ks = (k.astype(np.float32) / lam.view(np.float16).astype(np.float32)).astype(np.float64)
    ks = np.transpose(ks, (0, 2, 1, 3))
    step = c["ks"][:, :, :T].view(np.float16).astype(np.float64)[..., None]
    assert np.all(np.abs(kd - ks) <= step * 0.5 + 1e-6 * step)
    assert c["kq"].max() <= 15 and c["kz"].max() <= 15


def test_kv4_attention_against_library_softmax():
    """The attention over the dequantized cache equals numpy matmuls and a
    softmax written with numpy (library steps, independent of the C loops),
    for ragged lengths and grouped-query heads."""
    B, T, H, Hq, d = 3, 20, 2, 8, 128
    k, v = _kv_inputs(B, T, H, d, 8, k_outliers=[(11, 15.0)])
    lam = oracle.kv4_smooth_scales(k.reshape(B * T, H, d).view(np.uint16))
    c = oracle.kv4_quantize(k.view(np.uint16), v.view(np.uint16), lam, Tcap=24)
    q = np.random.default_rng(9).standard_normal((B, Hq, d)).astype(np.float16)
    lens = np.array([20, 1, 13], np.int32)
    o = oracle.kv4_decode_attention(q.view(np.uint16), lam, c, lens)
    kd, vd = _dequant(c, "k"), _dequant(c, "v")
    lf = lam.view(np.float16).astype(np.float32)
    for b in range(B):
        for hq in range(Hq):
            h = hq // (Hq // H)
            qs = (q[b, hq].astype(np.float32) * lf[h]).astype(np.float16).astype(np.float64)
            L = lens[b]
            sc = np.matmul(kd[b, h, :L], qs) / np.sqrt(d)
            p = np.exp(sc - sc.max())
            p /= p.sum()
            np.testing.assert_allclose(o[b, hq], np.matmul(p, vd[b, h, :L]), rtol=1e-10, atol=1e-12)
    # one token: the output is that token's dequantized value vector
    np.testing.assert_allclose(o[1, 0], vd[1, 0, 0], rtol=0, atol=1e-15)


def test_kv4_attention_two_token_closed_form():
    """Two tokens whose keys sit exactly on the 4-bit grid: the output is the
    logistic weighting of the two value vectors, in closed form."""
    import math
    d = 128
    k = np.zeros((1, 2, 1, d), np.float16)
    v = np.zeros((1, 2, 1, d), np.float16)
    k[0, 0, 0, 0], k[0, 1, 0, 0] = 0.9375, -0.9375  # 15/16: scale 1/16, codes 15 / 0
    v[0, 0, 0, 1] = 1.875                         # 15/8: scale 1/8, code 15
    calib = np.ones((1, 1, d), np.float16)        # lambda = sqrt(1) = 1
    lam = oracle.kv4_smooth_scales(calib.view(np.uint16))
    c = oracle.kv4_quantize(k.view(np.uint16), v.view(np.uint16), lam)
    assert c["ks"][0, 0, 0] == np.float16(0.0625).view(np.uint16) and c["kq"][0, 0, 0, 0] == 15
    assert c["kz"][0, 0, 1] == 15 and c["kq"][0, 0, 1, 0] == 0
    q = np.zeros((1, 1, d), np.float16)
    q[0, 0, 0] = 1.0
    o = oracle.kv4_decode_attention(q.view(np.uint16), lam, c, [2])
    want = 1.875 / (1.0 + math.exp(-2 * 0.9375 / math.sqrt(d)))
    assert abs(o[0, 0, 1] - want) <= 1e-15 * want
    assert np.all(o[0, 0, [0] + list(range(2, d))] == 0)


def test_smoothing_reduces_kv4_attention_error_with_key_outliers():
    """The pages' claim for SmoothAttention on synthetic keys with outlier
    channels: with the scales the KV4 attention is closer to the FP16 attention
    than without them (lambda = 1)."""
    for outliers, ratio in (([(5, 10.0)], 0.6), ([(5, 25.0), (77, 18.0), (100, 30.0)], 0.8)):
        errs = _kv4_errors_with_and_without_smoothing(outliers)
        assert errs[0] < errs[1] * ratio, (outliers, errs)


def _kv4_errors_with_and_without_smoothing(outliers):
    B, T, H, Hq, d = 2, 256, 2, 4, 128
    k, v = _kv_inputs(B, T, H, d, 10, k_outliers=outliers)
    q = np.random.default_rng(11).standard_normal((B, Hq, d)).astype(np.float16)
    lens = np.array([T, T], np.int32)
    kf, vf = k.astype(np.float64), v.astype(np.float64)
    ref = np.zeros((B, Hq, d))
    for b in range(B):
        for hq in range(Hq):
            h = hq // (Hq // H)
            sc = kf[b, :, h] @ q[b, hq].astype(np.float64) / np.sqrt(d)
            p = np.exp(sc - sc.max())
            ref[b, hq] = (p / p.sum()) @ vf[b, :, h]
    errs = []
    for lam in (oracle.kv4_smooth_scales(k.reshape(B * T, H, d).view(np.uint16)),
                np.full((H, d), np.float16(1.0).view(np.uint16), np.uint16)):
        c = oracle.kv4_quantize(k.view(np.uint16), v.view(np.uint16), lam)
        o = oracle.kv4_decode_attention(q.view(np.uint16), lam, c, lens)
        errs.append(np.linalg.norm(o - ref) / np.linalg.norm(ref))
    return errs


# --- RMSNorm producer (reading R17) ------------------------------------------

def _rms_rows(rng, M, K, wide=True):
    """FP16 rows; with wide=True they mix subnormals, ordinary values, zeros and
    values near the FP16 maximum, so the exact sum of squares spans its range."""
    x = rng.standard_normal((M, K)).astype(np.float32)
    if wide:
        e = rng.integers(-24, 16, size=(M, K)).astype(np.float32)
        x = np.sign(x) * np.exp2(e) * rng.uniform(1.0, 1.99, size=(M, K)).astype(np.float32)
        x[rng.random((M, K)) < 0.1] = 0.0
        x = np.clip(x, -65504, 65504)
    return x.astype(np.float16)


def _exact_r(x16, eps):
    """1 / sqrt(S/K + eps) from the exact sum of squares S (Python fractions)."""
    from fractions import Fraction
    out = []
    for row in x16.astype(np.float64):
        S = sum(Fraction(float(v)) ** 2 for v in row)
        out.append(1.0 / np.sqrt(float(S / len(row)) + float(eps)))
    return np.array(out)


@pytest.mark.parametrize("K,wide", [(1, True), (3, True), (128, True), (4096, True), (4096, False)])
def test_rmsnorm_scale_and_outputs_within_rounding_of_exact(K, wide):
    """r is within a few fp32 roundings of 1/sqrt(mean(x^2) + eps) computed from
    the exact sum of squares (which pins the 128-bit sum over subnormals and
    values near 65504 alike), and each y within half an FP16 step of
    x * gamma * r_exact plus those roundings."""
    rng = np.random.default_rng(900 + K)
    M = 6
    x = _rms_rows(rng, M, K, wide)
    gamma = rng.uniform(0.25, 2.0, size=K).astype(np.float16)
    eps = np.float32(1e-5)
    y, r = oracle.rmsnorm(x.view(np.uint16), gamma.view(np.uint16), float(eps), want_r=True)
    r_ex = _exact_r(x, eps)
    assert np.all(np.abs(r.astype(np.float64) - r_ex) <= r_ex * 2.0**-21)
    want = x.astype(np.float64) * gamma.astype(np.float64)[None] * r_ex[:, None]
    got = y.view(np.float16).astype(np.float64)
    half_step = 0.5 * np.spacing(np.abs(want).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(got - want) <= half_step + np.abs(want) * 2.0**-20)


def test_rmsnorm_power_of_two_invariance():
    """Scaling a row by 2^j scales S by 4^j and r by 2^-j exactly (every step
    rounds the same way at another exponent), so y does not change at all."""
    rng = np.random.default_rng(910)
    x = rng.uniform(0.05, 50.0, size=(5, 512)).astype(np.float32)
    x *= np.where(rng.random(x.shape) < 0.5, -1.0, 1.0)
    x16 = x.astype(np.float16)
    gamma = rng.uniform(0.5, 1.5, size=512).astype(np.float16).view(np.uint16)
    y0 = oracle.rmsnorm(x16.view(np.uint16), gamma, 1e-30)
    for j in (-3, 4):
        xs = (x16.astype(np.float32) * np.float32(2.0**j)).astype(np.float16)
        assert np.array_equal(xs.astype(np.float32), x16.astype(np.float32) * np.float32(2.0**j))
        np.testing.assert_array_equal(oracle.rmsnorm(xs.view(np.uint16), gamma, 1e-30), y0)


@pytest.mark.parametrize("K", [128, 4096, 14336])
def test_rmsnorm_single_input_closed_form(K):
    """One nonzero input a: mean(x^2) = a^2 / K, so y = sign(a) sqrt(K) gamma at
    that position (to FP16 and fp32 rounding) and 0 elsewhere."""
    x = np.zeros((3, K), np.float16)
    x[0, 5], x[1, K - 1], x[2, 0] = 3.5, -0.001, 1000.0
    gamma = np.full(K, np.float16(0.5))
    y = oracle.rmsnorm(x.view(np.uint16), gamma.view(np.uint16), 1e-30).view(np.float16)
    for m, (pos, sgn) in enumerate([(5, 1), (K - 1, -1), (0, 1)]):
        want = sgn * np.sqrt(K) * 0.5
        assert abs(float(y[m, pos]) - want) <= abs(want) * 2.0**-10
        assert np.count_nonzero(y[m].astype(np.float32)) == 1


def test_rmsnorm_rejects_bad_eps():
    x = np.zeros((1, 128), np.uint16)
    g = np.zeros(128, np.uint16)
    for eps in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(Exception):
            oracle.rmsnorm(x, g, eps)
