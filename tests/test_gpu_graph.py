"""The hot path replayed from a captured HIP graph (torch.cuda.CUDAGraph): the decode step
(kvq_quantize, kvq_dequantize, kvq_score_decode) and the RRS chain (kvq_rrs_smooth_scales,
kvq_rrs_quantize_act, kvq_rrs_quantize_weights, kvq_rrs_gemm) enqueue only kernels (no memset
nodes, no allocation), so a captured graph reproduces the eager results on every replay.  Each
replay follows eager work on other buffers and a poisoning of the graph's outputs, and must give
the eager outputs byte for byte."""
import numpy as np
import pytest
import torch

from activation_quantization_amd import kvq, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _poison(ts):
    for t in ts:
        if t is not None:
            t.view(torch.uint8).fill_(0xCD)


def _same(a, b):
    return a is None and b is None or torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_decode_step_replays_from_a_graph():
    S, T, H, G, D = 2, 512, 2, 4, 128
    d = kvq.Desc(S, T, H, D, 4, "nsep_pchan", 128, 128, torch.float16)
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal((S * T, H, D)).astype(np.float16)).to(DEV)
    x2 = torch.from_numpy(rng.standard_normal((S * T, H, D)).astype(np.float16)).to(DEV)
    q = torch.from_numpy(rng.standard_normal((S, H * G, D)).astype(np.float16)).to(DEV)
    sg = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=(H, D))).to(DEV)

    def step(out, y, sc):
        kvq.quantize(d, x, sg, out=out)
        kvq.dequantize(d, *out, sg, out=y)
        kvq.score_decode(d, q, *out, sg, out=sc)

    ref = kvq.alloc_outputs(d, DEV)
    ref_y = torch.empty_like(x)
    ref_sc = torch.empty((S, H * G, T), dtype=torch.float32, device=DEV)
    step(ref, ref_y, ref_sc)
    out = kvq.alloc_outputs(d, DEV)
    y = torch.empty_like(x)
    sc = torch.empty_like(ref_sc)
    side = kvq.alloc_outputs(d, DEV)
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        step(out, y, sc)                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        step(out, y, sc)
    for rep in range(3):
        kvq.quantize(d, x2, sg, out=side)                  # eager work between replays
        _poison((*out, y, sc))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert _same(a, b), f"replay {rep}: quantize outputs differ"
        assert _same(y, ref_y), f"replay {rep}: dequantize differs"
        assert _same(sc, ref_sc), f"replay {rep}: scores differ"


def test_rrs_chain_replays_from_a_graph():
    n, m, k = 256, 192, 1024
    rng = np.random.default_rng(4)
    xa = rng.standard_normal((n, k)).astype(np.float32)
    xa[:, 7] *= 50.0
    x = torch.from_numpy(xa).to(torch.bfloat16).to(DEV)
    x2 = (x * 2).contiguous()
    w = synth.make_weights(m, k, seed=5, dtype="bf16").to(DEV)
    sg = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=k)).to(DEV)

    s0 = kvq.rrs_smooth_scales(x, sg, 128)
    xq0 = kvq.rrs_quantize_act(x, sg, 128, s0, 4)
    wq0 = kvq.rrs_quantize_weights(w, sg, 128, 4)
    y0 = kvq.rrs_gemm(*xq0, *wq0, s0)
    s = torch.empty_like(s0)
    xq = tuple(torch.empty_like(t) for t in xq0)
    wq = tuple(torch.empty_like(t) for t in wq0)
    y = torch.empty_like(y0)
    s_side = torch.empty_like(s0)

    def chain():
        kvq.rrs_smooth_scales(x, sg, 128, out=s)
        kvq.rrs_quantize_act(x, sg, 128, s, 4, out=xq)
        kvq.rrs_quantize_weights(w, sg, 128, 4, out=wq)
        kvq.rrs_gemm(*xq, *wq, s, out=y)

    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        chain()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        chain()
    for rep in range(3):
        kvq.rrs_smooth_scales(x2, sg, 128, out=s_side)     # eager work between replays
        _poison((s, *xq, *wq, y))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(s, s0), f"replay {rep}: smoothing scales differ"
        for a, b in zip((*xq, *wq), (*xq0, *wq0)):
            assert _same(a, b), f"replay {rep}: codes or scales differ"
        assert _same(y, y0), f"replay {rep}: gemm output differs"
