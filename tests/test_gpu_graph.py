"""Every entry point of the per-call path captured in one HIP graph: each
replay, with fresh inputs copied into the captured buffers eagerly in between,
gives the same bits as the eager calls on those inputs (the library launches
kernels only: no allocation, no memset, no host synchronization)."""
import pytest
import torch

import quantized_gemm_qoq_amd as qoq
from quantized_gemm_qoq_amd import workloads

from gpu_util import DEV

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

# (M, K, N) GEMMs on each kernel: streaming decode, split-K 16-row waves,
# LDS-pipelined, wide
GEMMS = [(64, 1024, 768), (200, 1664, 272), (600, 1152, 528), (640, 640, 16400)]


def _f16(shape, seed, scale):
    return workloads.random_fp16(shape, seed, scale).to(DEV)


def test_graph_replays_match_eager_calls():
    torch.manual_seed(0)
    packed = {}
    for i, (M, K, N) in enumerate(GEMMS):
        w = _f16((N, K), 900 + i, 0.02)
        for mode in ("g128", "per_channel", "w8a8"):
            packed[(i, mode)] = qoq.PackedWeight(mode, w)
    gamma = _f16((1024,), 950, 0.5).abs() + 0.5
    lam = qoq.qoq_kv4_smooth_scales(_f16((96, 4, 128), 951, 1.0))
    cache = qoq.KV4Cache(3, 4, 96, DEV, lam)
    cache.append(_f16((3, 96, 4, 128), 952, 1.0), _f16((3, 96, 4, 128), 953, 1.0), 0)
    need_att = int(qoq.load_library().qoq_kv4_attention_workspace_bytes(3, 16, 4, 128, 96))
    ws_att = torch.empty((max(need_att, 16),), dtype=torch.uint8, device=DEV)

    # static inputs
    xs = [torch.empty((M, K), dtype=torch.float16, device=DEV) for (M, K, N) in GEMMS]
    gu = torch.empty((16, 2 * 12288), dtype=torch.float16, device=DEV)
    xn = torch.empty((64, 1024), dtype=torch.float16, device=DEV)
    q = torch.empty((3, 16, 128), dtype=torch.float16, device=DEV)
    lens = torch.empty((3,), dtype=torch.int32, device=DEV)

    def fill(r):
        for i, (M, K, N) in enumerate(GEMMS):
            xs[i].copy_(_f16((M, K), 1000 + 10 * r + i, 1.0))
        gu.copy_(_f16(tuple(gu.shape), 1100 + r, 2.0))
        xn.copy_(_f16(tuple(xn.shape), 1200 + r, 1.0))
        q.copy_(_f16(tuple(q.shape), 1300 + r, 1.0))
        lens.copy_(torch.tensor([96, 17 + r, 50], dtype=torch.int32))

    def outputs():
        return {"y": {k: torch.empty((GEMMS[k[0]][0], GEMMS[k[0]][2]), dtype=torch.float16, device=DEV)
                      for k in packed},
                "silu": (torch.empty((qoq.qoq_act_bytes(16, 12288),), dtype=torch.int8, device=DEV),
                         torch.empty((16,), dtype=torch.float16, device=DEV),
                         torch.empty((16,), dtype=torch.int32, device=DEV)),
                "rms": (torch.empty((qoq.qoq_act_bytes(64, 1024),), dtype=torch.int8, device=DEV),
                        torch.empty((64,), dtype=torch.float16, device=DEV),
                        torch.empty((64,), dtype=torch.int32, device=DEV)),
                "att": torch.empty((3, 16, 128), dtype=torch.float16, device=DEV)}

    ws_silu = torch.empty((int(qoq.load_library().qoq_silu_mul_workspace_bytes(16, 12288)),),
                          dtype=torch.uint8, device=DEV)
    assert ws_silu.numel() > 0

    def step(out):
        for (i, mode), pw in packed.items():
            pw.forward(xs[i], y=out["y"][(i, mode)])
        qoq.qoq_silu_mul_quantize_act(gu, *out["silu"], workspace=ws_silu)
        qoq.qoq_rmsnorm_quantize_act(xn, gamma, 1e-5, *out["rms"])
        cache.attention(q, lens, o=out["att"], workspace=ws_att)

    fill(0)
    captured = outputs()
    step(captured)  # warm-up outside the graph
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(captured)
    for r in range(1, 4):
        fill(r)
        eager = outputs()
        step(eager)
        torch.cuda.synchronize()
        before = {k: captured["y"][k].clone() for k in packed}
        before_att = captured["att"].clone()
        graph.replay()
        torch.cuda.synchronize()
        print(f"graph replay {r}", flush=True)
        for k in packed:
            assert torch.equal(captured["y"][k], eager["y"][k]), (r, k)
        for name in ("silu", "rms"):
            for a, b in zip(captured[name], eager[name]):
                assert torch.equal(a, b), (r, name)
        assert torch.equal(captured["att"], eager["att"]), r
        # the replay rewrote every output (its inputs differ from the last round's)
        assert not torch.equal(captured["att"], before_att), r
        for k in packed:
            assert not torch.equal(captured["y"][k], before[k]), (r, k)


def test_captured_split_call_survives_workspace_growth():
    """A graph that captured a split-K call on its stream's shared workspace
    still replays correctly after a later call on the same stream needed a
    larger workspace: the smaller one stays allocated, so tensors allocated
    afterwards neither receive the replay's partial sums nor feed it."""
    small, large = (200, 1664, 272), (128, 8192, 24576)  # (M, K, N)
    need_small = qoq.qoq_gemm_workspace_bytes("g128", small[0], small[2], small[1])
    assert 0 < need_small < qoq.qoq_gemm_workspace_bytes("g128", large[0], large[2], large[1])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        (M, K, N) = small
        pw = qoq.PackedWeight("g128", _f16((N, K), 970, 0.02))
        x = _f16((M, K), 971, 1.0)
        xq, s_x, _ = qoq.qoq_quantize_act(x, want_rowsum=False)
        want = qoq.qoq_w4a8_gemm("g128", xq, s_x, None, pw.blob, pw.s_c, N)
        y = torch.empty_like(want)
        qoq.qoq_w4a8_gemm("g128", xq, s_x, None, pw.blob, pw.s_c, N, y=y)  # warm-up on this stream
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            qoq.qoq_w4a8_gemm("g128", xq, s_x, None, pw.blob, pw.s_c, N, y=y)
        (M2, K2, N2) = large
        pw2 = qoq.PackedWeight("g128", _f16((N2, K2), 972, 0.02))
        xq2, s_x2, _ = qoq.qoq_quantize_act(_f16((M2, K2), 973, 1.0), want_rowsum=False)
        qoq.qoq_w4a8_gemm("g128", xq2, s_x2, None, pw2.blob, pw2.s_c, N2)  # grows the workspace
        s.synchronize()
        del pw2, xq2, s_x2
        torch.cuda.empty_cache()
        need = need_small
        fillers = [torch.full((max(need, 1 << 20),), 0x55, dtype=torch.uint8, device=DEV) for _ in range(8)]
        for r in range(3):
            y.fill_(0)
            g.replay()
            s.synchronize()
            assert torch.equal(y, want), r
        s.synchronize()
        for f in fillers:
            assert bool((f == 0x55).all())
