"""GPU parity of KV4 decode attention with SmoothAttention against the CPU
oracle, through the C ABI.

Bit-exact: the smoothing scales (every FP16 value as a channel maximum), the
4-bit key and value codes, their scales and zeros, also when a cache is filled
by several appends. The attention output (FP16 products with FP32 sums in the
kernel's own order, then FP16) within half an FP16 ulp plus 1e-4 of the largest
|o| of its (sequence, head) of the oracle's fp64 value on the same cache.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_qoq_amd as qoq

from gpu_util import DEV, f16_dev, host, host_bits, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

D = 128


def _kv(B, T, H, seed, outliers=((5, 20.0), (77, 12.0))):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, T, H, D)).astype(np.float32)
    for ch, f in outliers:
        k[..., ch] *= f
    v = rng.standard_normal((B, T, H, D)).astype(np.float32)
    return k.astype(np.float16), v.astype(np.float16)


def _gpu_cache_as_oracle(cache, T):
    """The GPU cache (two codes per byte, values in 16-token blocks) in the
    oracle's layout (one code per byte, token-major), for the first T tokens."""
    kq = host(cache.kq)[:, :, :T]
    k = np.stack([kq & 15, kq >> 4], axis=-1).reshape(*kq.shape[:3], D)
    vb = host(cache.vq)  # [B, H, Tcap/16, 64, 16]
    vb = np.transpose(vb, (0, 1, 2, 4, 3)).reshape(vb.shape[0], vb.shape[1], -1, 64)[:, :, :T]
    v = np.stack([vb & 15, vb >> 4], axis=-1).reshape(*vb.shape[:3], D)
    return {"kq": k, "vq": v,
            "ks": host_bits(cache.ks)[:, :, :T], "vs": host_bits(cache.vs)[:, :, :T],
            "kz": host(cache.kz)[:, :, :T], "vz": host(cache.vz)[:, :, :T]}


def test_smooth_scales_every_fp16_maximum():
    vals = np.arange(1, 0x7C00, dtype=np.uint16)
    H = (vals.size + D - 1) // D
    k = np.zeros((3, H * D), np.uint16)
    k[0, : vals.size] = vals
    k[1, : vals.size] = vals | 0x8000        # the negative of the maximum
    k[2, : vals.size] = vals >> 1            # smaller
    k = k.reshape(3, H, D)
    print(f"kv4 smoothing scales over {vals.size} maxima", flush=True)
    lam = qoq.qoq_kv4_smooth_scales(f16_dev(k))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(lam), oracle.kv4_smooth_scales(k))


@pytest.mark.parametrize("B,T,H,Tcap", [(1, 1, 1, 16), (3, 40, 4, 48), (2, 300, 8, 304)])
def test_append_matches_oracle(B, T, H, Tcap):
    k, v = _kv(B, T, H, 400 + T)
    if T > 3:
        k[0, 2] = 0  # an all-zero key: scale 0, codes 0
        v[0, 3] = np.float16(0.5)  # a constant value vector
    lam_w = oracle.kv4_smooth_scales(k.reshape(B * T, H, D).view(np.uint16))
    want = oracle.kv4_quantize(k.view(np.uint16), v.view(np.uint16), lam_w)
    print(f"kv4 append B={B} T={T} H={H} Tcap={Tcap}", flush=True)
    lam = qoq.qoq_kv4_smooth_scales(f16_dev(k.reshape(B * T, H, D).view(np.uint16)))
    cache = qoq.KV4Cache(B, H, Tcap, DEV, lam)
    cache.append(f16_dev(k.view(np.uint16)), f16_dev(v.view(np.uint16)), 0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(lam), lam_w)
    got = _gpu_cache_as_oracle(cache, T)
    for key in ("kq", "vq", "ks", "vs", "kz", "vz"):
        np.testing.assert_array_equal(got[key], want[key], err_msg=key)
    if T > 1:
        # the same cache filled by two appends (the second starts mid-block)
        c2 = qoq.KV4Cache(B, H, Tcap, DEV, lam)
        t1 = T // 2 + 1
        c2.append(f16_dev(np.ascontiguousarray(k[:, :t1]).view(np.uint16)),
                  f16_dev(np.ascontiguousarray(v[:, :t1]).view(np.uint16)), 0)
        c2.append(f16_dev(np.ascontiguousarray(k[:, t1:]).view(np.uint16)),
                  f16_dev(np.ascontiguousarray(v[:, t1:]).view(np.uint16)), t1)
        torch.cuda.synchronize()
        for name in ("kq", "vq", "ks", "vs", "kz", "vz"):
            assert torch.equal(getattr(c2, name), getattr(cache, name)), name


def _assert_attn_close(o_bits, ref, what=""):
    o = np.asarray(o_bits).view(np.float16).astype(np.float64)
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    err = np.abs(o - ref)
    bound = 0.5 * ulp + 1e-4 * scale + 1e-12
    assert np.all(err <= bound), (what, float((err / bound).max()))


@pytest.mark.parametrize("B,Hq,H,Tcap,lens", [
    (2, 8, 8, 32, [32, 17]),
    (3, 32, 8, 96, [96, 1, 50]),
    (2, 16, 8, 304, [300, 16]),
    (1, 8, 4, 1536, [1536]),           # many chunks
    (4, 64, 8, 512, [512, 400, 2, 257]),
    (2, 4, 4, 64, [0, 64]),            # an empty sequence gives zeros
])
def test_decode_attention_matches_oracle(B, Hq, H, Tcap, lens):
    k, v = _kv(B, Tcap, H, 500 + Tcap + Hq)
    lam_w = oracle.kv4_smooth_scales(k.reshape(B * Tcap, H, D).view(np.uint16))
    cache_w = oracle.kv4_quantize(k.view(np.uint16), v.view(np.uint16), lam_w)
    q = np.random.default_rng(600 + Hq).standard_normal((B, Hq, D)).astype(np.float16)
    print(f"kv4 attention B={B} Hq={Hq} H={H} Tcap={Tcap} lens={lens}", flush=True)
    lam = to_dev(lam_w, torch.float16)
    cache = qoq.KV4Cache(B, H, Tcap, DEV, lam)
    cache.append(f16_dev(k.view(np.uint16)), f16_dev(v.view(np.uint16)), 0)
    d_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = cache.attention(f16_dev(q.view(np.uint16)), d_lens)
    ws = torch.full((qoq.load_library().qoq_kv4_attention_workspace_bytes(B, Hq, H, D, Tcap),),
                    0x7F, dtype=torch.uint8, device=DEV)  # junk: no initialisation needed
    o2 = cache.attention(f16_dev(q.view(np.uint16)), d_lens, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    ref = np.zeros((B, Hq, D))
    live = [b for b in range(B) if lens[b] > 0]
    if live:
        sub = {key: val[live] for key, val in cache_w.items()}
        ref[live] = oracle.kv4_decode_attention(q[live].view(np.uint16), lam_w, sub,
                                                np.array(lens, np.int32)[live])
    ob = host_bits(o)
    _assert_attn_close(ob, ref, "attention")
    for b in range(B):
        if lens[b] == 0:
            assert not ob[b].any()


def test_decode_attention_magnitudes():
    """Queries from 1e-4 to 30 times unit size (flat to one-hot attention) and
    value vectors whose ranges span four decades along the sequence, large ones
    late: the kernel's power-of-two scalings of queries and weights and its
    running maximum all move."""
    B, Hq, H, Tcap = 2, 16, 4, 1024
    lens = [1024, 700]
    k, v = _kv(B, Tcap, H, 810)
    rng = np.random.default_rng(811)
    vf = 10.0 ** np.linspace(-3.0, 1.0, Tcap) * rng.uniform(0.5, 1.0, Tcap)
    v = (v.astype(np.float32) * vf[None, :, None, None].astype(np.float32)).astype(np.float16)
    qf = np.array([1e-4, 1e-2, 1.0, 3.0, 10.0, 30.0, 0.3, 1.0] * 2, np.float32)
    q = (rng.standard_normal((B, Hq, D)).astype(np.float32) * qf[None, :, None]).astype(np.float16)
    lam_w = oracle.kv4_smooth_scales(k.reshape(B * Tcap, H, D).view(np.uint16))
    cache_w = oracle.kv4_quantize(k.view(np.uint16), v.view(np.uint16), lam_w)
    print("kv4 attention magnitudes", flush=True)
    cache = qoq.KV4Cache(B, H, Tcap, DEV, to_dev(lam_w, torch.float16))
    cache.append(f16_dev(k.view(np.uint16)), f16_dev(v.view(np.uint16)), 0)
    o = cache.attention(f16_dev(q.view(np.uint16)), torch.tensor(lens, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    ref = oracle.kv4_decode_attention(q.view(np.uint16), lam_w, cache_w, np.array(lens, np.int32))
    _assert_attn_close(host_bits(o), ref, "magnitudes")


def test_decode_attention_serving_shape():
    """Llama-3-8B decode at the pages' serving point (1024 input + 512 output
    tokens: the cache holds 1536 at the last step), 64 sequences, 32 query and 8
    KV heads, ragged lengths; checked at sampled (sequence, head) pairs."""
    B, Hq, H, Tcap = 64, 32, 8, 1536
    rng = np.random.default_rng(700)
    lens = rng.integers(1024, Tcap + 1, size=B).astype(np.int32)
    lens[0] = Tcap
    k, v = _kv(B, Tcap, H, 701)
    lam_w = oracle.kv4_smooth_scales(k[:4].reshape(4 * Tcap, H, D).view(np.uint16))
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    print("kv4 attention serving shape", flush=True)
    cache = qoq.KV4Cache(B, H, Tcap, DEV, to_dev(lam_w, torch.float16))
    cache.append(f16_dev(k.view(np.uint16)), f16_dev(v.view(np.uint16)), 0)
    o = cache.attention(f16_dev(q.view(np.uint16)), torch.from_numpy(lens).to(DEV))
    torch.cuda.synchronize()
    ob = host_bits(o)
    got = _gpu_cache_as_oracle(cache, Tcap)
    for b in (0, 17, 63):
        want = oracle.kv4_quantize(k[b:b + 1].view(np.uint16), v[b:b + 1].view(np.uint16), lam_w)
        for key in ("kq", "vq", "ks", "kz"):
            np.testing.assert_array_equal(got[key][b:b + 1], want[key], err_msg=key)
        ref = oracle.kv4_decode_attention(q[b:b + 1].view(np.uint16), lam_w, want, lens[b:b + 1])
        _assert_attn_close(ob[b:b + 1], ref, f"sequence {b}")
