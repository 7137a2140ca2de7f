"""Pin the oracle to hand-worked examples of the pages' equations.

Each fixture under tests/golden/ holds inputs whose scales are powers of two, so
that every expected value was derived by hand (the derivations are in the
fixtures). Several entries sit exactly on rounding ties, which pins
round-half-to-even; the group examples pin the integer group scale, zero and
code formulas of the stage-2 equation; the GEMM example pins the contraction
and the one-time rescale.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16_bits(values):
    return np.asarray(values, dtype=np.float16).view(np.uint16)


def _act_inputs():
    d = _load("act_quant.json")
    K = d["K"]
    x = np.zeros((len(d["rows"]), K), np.float16)
    for r, row in enumerate(d["rows"]):
        for k, v in row["nonzero"].items():
            x[r, int(k)] = v
    return d, x.view(np.uint16)


def test_act_quant_golden():
    d, x = _act_inputs()
    xq, s_x, rowsum = oracle.quantize_act(x)
    for r, row in enumerate(d["rows"]):
        want = np.zeros(d["K"], np.int8)
        for k, v in row["xq_nonzero"].items():
            want[int(k)] = v
        assert s_x[r] == row["s_x_bits"], (r, s_x[r])
        np.testing.assert_array_equal(xq[r], want)
        assert rowsum[r] == row["rowsum"]


def _g128_inputs():
    d = _load("weights_g128.json")
    K = d["K"]
    rows = []
    for row in d["rows"]:
        w8 = np.zeros(K, np.int64)
        for k, v in row["w8_nonzero"].items():
            w8[int(k)] = v
        rows.append(w8.astype(np.float64) * 2.0 ** row["s_c_pow2"])
    w = np.array(rows).astype(np.float16)
    # The inputs are exact: w8 * 2^e with |w8| <= 119 fits an FP16 significand.
    assert np.array_equal(w.astype(np.float64), np.array(rows))
    return d, w.view(np.uint16)


def test_weights_g128_golden():
    d, w = _g128_inputs()
    out = oracle.quantize_weights(oracle.MODE_G128, w, want_w8=True)
    for r, row in enumerate(d["rows"]):
        assert out["s_c"][r] == row["s_c_bits"]
        w8 = np.zeros(d["K"], np.int8)
        for k, v in row["w8_nonzero"].items():
            w8[int(k)] = v
        np.testing.assert_array_equal(out["w8"][r], w8)
        for g, grp in enumerate(row["groups"]):
            assert out["s_g"][r, g] == grp["s_g"], (r, g)
            assert out["z"][r, g] == grp["z"], (r, g)
            for k, v in grp["q_at"].items():
                assert out["q"][r, int(k)] == v, (r, k)


def _pc_inputs():
    d = _load("weights_per_channel.json")
    K = d["K"]
    w = np.zeros((len(d["rows"]), K), np.uint16)
    for r, row in enumerate(d["rows"]):
        for k, v in row.get("w_nonzero", {}).items():
            w[r, int(k)] = _f16_bits([v])[0]
        for k, v in row.get("w_nonzero_bits", {}).items():
            w[r, int(k)] = v
    return d, w


def test_weights_per_channel_golden():
    d, w = _pc_inputs()
    out = oracle.quantize_weights(oracle.MODE_PER_CHANNEL, w)
    for r, row in enumerate(d["rows"]):
        assert out["s_c"][r] == row["s_c_bits"], (r, out["s_c"][r])
        assert out["z"][r] == row["z"]
        for k, v in row["q_at"].items():
            assert out["q"][r, int(k)] == v, (r, k)


def _xq_from(nonzero_rows, K):
    xq = np.zeros((len(nonzero_rows), K), np.int8)
    for r, row in enumerate(nonzero_rows):
        for k, v in row.items():
            xq[r, int(k)] = v
    return xq


def test_gemm_g128_golden():
    g = _load("gemm.json")["g128"]
    _, w = _g128_inputs()
    wq = oracle.quantize_weights(oracle.MODE_G128, w)
    xq = _xq_from(g["xq_nonzero"], g["K"])
    acc = oracle.gemm(oracle.MODE_G128, xq, wq["q"], wq["s_g"], wq["z"])
    np.testing.assert_array_equal(acc, np.array(g["acc"], np.int32))
    y = oracle.epilogue(acc, np.array(g["s_x_bits"], np.uint16), wq["s_c"])
    np.testing.assert_array_equal(y, np.array(g["y"]))  # exact: powers of two


def test_gemm_per_channel_golden():
    g = _load("gemm.json")["per_channel"]
    _, w = _pc_inputs()
    wq = oracle.quantize_weights(oracle.MODE_PER_CHANNEL, w[:2])
    xq = _xq_from(g["xq_nonzero"], g["K"])
    acc = oracle.gemm(oracle.MODE_PER_CHANNEL, xq, wq["q"], None, wq["z"])
    np.testing.assert_array_equal(acc, np.array(g["acc"], np.int32))
    assert int(xq.astype(np.int64).sum()) == g["rowsum"][0]
    y = oracle.epilogue(acc, np.array(g["s_x_bits"], np.uint16), wq["s_c"])
    np.testing.assert_array_equal(y, np.array(g["y"]))


def test_pack_layout_golden():
    d = _load("pack_layout.json")
    N, K = d["N"], d["K"]
    q = np.zeros((N, K), np.uint8)
    for n, k, v in d["q_nonzero"]:
        q[n, k] = v
    s_g = np.ones((N, K // 128), np.uint8)
    z = np.zeros((N, K // 128), np.uint8)
    for n, g, sg, zz in d["s_g_z_nonzero"]:
        s_g[n, g] = sg
        z[n, g] = zz
    blob = oracle.pack(oracle.MODE_G128, q, s_g, z)
    assert blob.size == d["total_bytes"] == oracle.packed_bytes(oracle.MODE_G128, N, K)
    want = np.zeros(d["total_bytes"], np.uint8)
    for off, v in d["bytes_nonzero"].items():
        want[int(off)] = v
    np.testing.assert_array_equal(blob, want)


def test_per_channel_pack_size():
    # codes N*K/2 plus one zero byte per channel
    assert oracle.packed_bytes(oracle.MODE_PER_CHANNEL, 32, 256) == 32 * 128 + 32
    # g128: one parameter byte per (channel, group)
    assert oracle.packed_bytes(oracle.MODE_G128, 32, 128 * 17) == 32 * 64 * 17 + 32 * 17
    assert oracle.packed_bytes(oracle.MODE_G128, 8, 128) == -1  # N must be a multiple of 16
    assert oracle.packed_bytes(oracle.MODE_G128, 16, 100) == -1  # K must be a multiple of 128


def test_pack_act_layout_hand_worked():
    """Packed activations (layout in include/qoq.h): with M = 17 (two row tiles,
    Mp = 32) and K = 256 (two groups), value (m, k) goes to
    (g * 2 + u) * 2048 + 1024 * s + 16 * (16 * j + r) + i."""
    xq = np.zeros((17, 256), np.int8)
    xq[0, 0] = 1     # g0 u0 s0 j0 r0 i0 -> 0
    xq[5, 77] = 2    # 77 = 64 + 13: s1 j0 i13; r5 -> 1024 + 80 + 13 = 1117
    xq[16, 130] = 3  # u1 r0, k 130: g1, kk 2 -> s0 j0 i2 -> (1*2 + 1)*2048 + 2 = 6146
    xq[15, 127] = -4  # u0 r15, kk 127: s1 j3 i15 -> 1024 + 16*(48 + 15) + 15 = 2047
    p = oracle.pack_act(xq)
    assert p.size == 32 * 256
    want = np.zeros(32 * 256, np.int8)
    want[0], want[1117], want[6146], want[2047] = 1, 2, 3, -4
    np.testing.assert_array_equal(p, want)


def _w8_inputs():
    d = _load("weights_w8.json")
    K = d["K"]
    rows = []
    for row in d["rows"]:
        w = np.zeros(K, np.float64)
        for k, v in row["w_nonzero_units"].items():
            w[int(k)] = v * 2.0 ** row["unit_pow2"]
        rows.append(w)
    w = np.array(rows)
    assert np.array_equal(w.astype(np.float16).astype(np.float64), w)  # exact in FP16
    return d, w.astype(np.float16).view(np.uint16)


def test_weights_w8_golden():
    d, w = _w8_inputs()
    s_c, q = oracle.quantize_weights_w8(w)
    for r, row in enumerate(d["rows"]):
        assert s_c[r] == row["s_c_bits"], (r, s_c[r])
        for k, v in row["q_at"].items():
            assert q[r, int(k)] == v, (r, k)
        # every entry not listed is zero in the input and in the codes
        listed = set(int(k) for k in row["w_nonzero_units"])
        rest = [k for k in range(d["K"]) if k not in listed]
        assert not q[r, rest].any()


def test_pack_w8_layout_golden():
    d = _load("pack_w8_layout.json")
    N, K = d["N"], d["K"]
    q = np.zeros((N, K), np.int8)
    for idx, (n, k, _, _) in enumerate(d["entries"]):
        q[n, k] = idx + 1
    blob = oracle.pack_w8(q)
    assert blob.size == N * K == oracle.w8_packed_bytes(N, K)
    want = np.zeros(N * K, np.uint8)
    for idx, (_, _, off, _) in enumerate(d["entries"]):
        want[off] = idx + 1
    np.testing.assert_array_equal(blob, want)


def test_w8_pack_size():
    assert oracle.w8_packed_bytes(16, 128) == 16 * 128
    assert oracle.w8_packed_bytes(8, 128) == -1
    assert oracle.w8_packed_bytes(16, 200) == -1


def test_w4a16_reproduces_hand_worked_w4a8_example():
    """W4A16 with FP16 activations X = s_x * xq (exact in FP16) must give the
    hand-worked W4A8 outputs of gemm.json: Y = s_c * sum_k X * W8^ =
    s_x * s_c * acc, the same exact values."""
    g = _load("gemm.json")["g128"]
    _, w = _g128_inputs()
    wq = oracle.quantize_weights(oracle.MODE_G128, w)
    xq = _xq_from(g["xq_nonzero"], g["K"]).astype(np.float64)
    s_x = np.array(g["s_x_bits"], np.uint16).view(np.float16).astype(np.float64)
    x = (xq * s_x[:, None]).astype(np.float16)
    assert np.array_equal(x.astype(np.float64), xq * s_x[:, None])
    y, absum = oracle.gemm_w4a16(oracle.MODE_G128, x.view(np.uint16), wq["s_c"], wq["q"],
                                 wq["s_g"], wq["z"])
    np.testing.assert_array_equal(y, np.array(g["y"]))
    assert np.all(absum >= np.abs(y))


def test_silu_mul_golden():
    """SiLU(gate) * up at the exponential's cut-offs and at zero, and the
    per-token quantization of the resulting row (hand-worked)."""
    d = _load("silu_mul.json")
    I = d["I"]
    gu = np.zeros((len(d["cases"]) + 1, 2 * I), np.float16)
    for r, c in enumerate(d["cases"]):
        gu[r, 0] = c["g"]
        gu[r, I] = c["u"]
    for k, c in enumerate(d["cases"]):  # the last row holds every case
        gu[-1, k] = c["g"]
        gu[-1, I + k] = c["u"]
    h, xq, s_x, rowsum = oracle.silu_mul_quantize_act(gu.view(np.uint16))
    for r, c in enumerate(d["cases"]):
        assert h[r, 0] == c["h_bits"], (r, h[r, 0])
    qr = d["quantized_row"]
    assert s_x[-1] == qr["s_x_bits"]
    want = np.zeros(I, np.int8)
    for k, v in qr["xq_nonzero"].items():
        want[int(k)] = v
    np.testing.assert_array_equal(xq[-1], want)
    assert rowsum[-1] == qr["rowsum"]


def _row(spec, K, dtype):
    v = np.full(K, spec.get("default", 0), dtype)
    if "even" in spec:
        v[0::2] = spec["even"]
        v[1::2] = spec["odd"]
    for k, val in spec.get("at", {}).items():
        v[int(k)] = val
    return v


def test_rmsnorm_golden():
    """RMSNorm rows whose sums of squares and means are exact, with the fp32
    square root, reciprocal and products rounded by hand (rmsnorm.json)."""
    d = _load("rmsnorm.json")
    K = d["K"]
    for c in d["cases"]:
        x = _row(c["x"], K, np.float16).view(np.uint16)[None]
        g = _row(c["gamma"], K, np.float16).view(np.uint16)
        y, r = oracle.rmsnorm(x, g, c["eps"], want_r=True)
        assert r.view(np.uint32)[0] == c["r_bits"], (c["name"], r.view(np.uint32)[0])
        np.testing.assert_array_equal(y[0], _row(c["y_bits"], K, np.uint16), err_msg=c["name"])
