"""GPU parity of the RRS INT4 GEMM path (kvq_rrs_smooth_scales, kvq_rrs_quantize_act,
kvq_rrs_quantize_weights, kvq_rrs_gemm) against the fp64 oracle through the C ABI.

Each entry point is compared on the inputs it is given: the smoothing scales with the oracle's
from the same activations; the activation codes and scales with the oracle's quantizer run on the
GPU's own smoothing scales; the GEMM with oracle.rrs_gemm of the GPU's own codes and scales.  The
whole chain is also compared end to end with the oracle's chain from the raw inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from activation_quantization_amd import kvq, synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL_S = 2e-6     # fp32 column maxima of an fp32 rotation against fp64
REL_Y = 1e-5     # fp32 sums of exact int32 group products against fp64, of max(|ref|, rms)


def _acts(seed, n, k, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, k)).astype(np.float32)
    x[:, rng.choice(k, size=max(1, k // 256), replace=False)] *= rng.uniform(30, 100)   # outlier channels
    x *= np.exp(0.5 * rng.standard_normal((n, 1))).astype(np.float32)                    # token swing
    return torch.from_numpy(x).to(dtype)


def _signs(seed, k):
    return torch.from_numpy(np.random.default_rng(seed + 1).choice(np.array([-1, 1], np.int8), size=k))


def _check_y(gpu, ref, what="y", rel=REL_Y):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    bad = np.abs(g - r) > rel * np.maximum(np.abs(r), rms)
    assert not np.any(bad), f"{what}: {int(bad.sum())} of {g.size} outside tolerance, first {np.argwhere(bad)[:3].tolist()}"


def _chain(x, w, sg, had, bits):
    xd, wd = x.to(DEV), w.to(DEV)
    sgd = sg.to(DEV) if had else None
    s = kvq.rrs_smooth_scales(xd, sgd, had)
    xc, xa = kvq.rrs_quantize_act(xd, sgd, had, s, bits)
    wc, wb = kvq.rrs_quantize_weights(wd, sgd, had, bits)
    y = kvq.rrs_gemm(xc, xa, wc, wb, s)
    torch.cuda.synchronize()
    return [t.cpu() for t in (s, xc, xa, wc, wb, y)]


@pytest.mark.parametrize("n,m,k,had,dtype,bits", [
    (200, 136, 256, 128, torch.bfloat16, 4),      # ragged rows and columns, two groups
    (129, 257, 512, 64, torch.float16, 4),
    (384, 128, 1024, 128, torch.bfloat16, 3),
    (64, 96, 128, 0, torch.float16, 4),           # one group, no rotation
    (300, 200, 4096, 128, torch.bfloat16, 4),     # the activation width: 32 groups
    (17, 33, 2048, 16, torch.float16, 2),
    (1, 1, 128, 0, torch.bfloat16, 4),            # one token, one output channel, one group
    (300, 1, 256, 32, torch.float16, 4),          # a single output channel
    (33, 40, 8192, 128, torch.float16, 4),        # the widest activations: 64 groups
])
def test_rrs_parity(n, m, k, had, dtype, bits):
    x = _acts(n + k, n, k, dtype)
    w = synth.make_weights(m, k, seed=m, dtype="bf16" if dtype == torch.bfloat16 else "f16")
    sg = _signs(k, k)
    s, xc, xa, wc, wb, y = _chain(x, w, sg, had, bits)
    sgn = sg.numpy() if had else None
    x64, w64 = x.double().numpy(), w.double().numpy()

    # smoothing scales
    s_ref = oracle.rrs_smooth_scales(x64, sgn, had)
    np.testing.assert_allclose(s.numpy(), s_ref, rtol=REL_S)
    # activation codes and scales, given the GPU's smoothing scales
    act = oracle.rrs_quantize_act(x64, sgn, had, s.double().numpy(), bits)
    parity.check_codes(xc.numpy(), act, bits)
    parity.check_rel_f16(xa.numpy(), act.scale, "activation scales")
    # weight codes and scales
    wq = oracle.rrs_quantize_weights(w64, sgn, had, bits)
    wref = oracle.Quantized(codes=wq.codes[:, 0, :], packed=None, v=wq.v[:, 0, :], nu=None, scale=wq.scale[:, 0],
                            norms16=None, scales16=wq.scales16[:, 0])
    parity.check_codes(wc.numpy(), wref, bits)
    parity.check_rel_f16(wb.numpy(), wref.scale, "weight scales")
    # the GEMM on the GPU's own codes and scales
    y_ref = oracle.rrs_gemm(oracle.unpack_nibbles(xc.numpy()), xa.numpy(), oracle.unpack_nibbles(wc.numpy()),
                            wb.numpy(), s.double().numpy())
    _check_y(y.numpy(), y_ref)
    # end to end against the oracle's chain from the raw inputs, its own smoothing scales included
    # (a code may differ at a rounding tie, and the fp16 scales may round differently by one ulp:
    # 1e-3 of the output's rms)
    act_ref = oracle.rrs_quantize_act(x64, sgn, had, s_ref, bits)
    y_chain = oracle.rrs_gemm(act_ref.codes, act_ref.scales16, wq.codes[:, 0, :], wq.scales16[:, 0], s_ref)
    _check_y(y.numpy(), y_chain, "end to end", rel=1e-3)


@pytest.mark.parametrize("n,k,had,dtype", [
    (2048 * 64 + 37, 128, 128, torch.bfloat16),   # 2049 tiles of 64 rows: several per resident workgroup, the last ragged
    (1030 * 32 + 5, 256, 64, torch.float16),      # two segments per token, an odd tail of rows
])
def test_rrs_smooth_scales_many_tiles(n, k, had, dtype):
    # the smoothing scales alone, over more 64-row tiles than the GPU holds workgroups at once
    x = _acts(n + 7, n, k, dtype)
    sg = _signs(k + 1, k)
    s = kvq.rrs_smooth_scales(x.to(DEV), sg.to(DEV), had)
    torch.cuda.synchronize()
    s_ref = oracle.rrs_smooth_scales(x.double().numpy(), sg.numpy(), had)
    np.testing.assert_allclose(s.cpu().numpy(), s_ref, rtol=REL_S)


def test_rrs_zero_rows_and_groups():
    # a zero activation row (a_t = 0, codes 0, y row 0) and a channel group that is zero in every
    # token (s_g = 0: its columns quantize to 0)
    n, m, k = 130, 140, 512
    x = _acts(5, n, k, torch.float16)
    x[7] = 0
    x[:, 128:256] = 0
    w = synth.make_weights(m, k, seed=3, dtype="f16")
    sg = _signs(9, k)
    s, xc, xa, wc, wb, y = _chain(x, w, sg, 128, 4)
    assert float(s[1]) == 0.0 and float(xa[7]) == 0.0
    assert not bool(xc[:, 64:128].any()) and not bool(xc[7].any())
    assert not bool(y[7].any())
    act = oracle.rrs_quantize_act(x.double().numpy(), sg.numpy(), 128, s.double().numpy(), 4)
    parity.check_codes(xc.numpy(), act, 4)
    y_ref = oracle.rrs_gemm(oracle.unpack_nibbles(xc.numpy()), xa.numpy(), oracle.unpack_nibbles(wc.numpy()),
                            wb.numpy(), s.double().numpy())
    _check_y(y.numpy(), y_ref)


def test_rrs_full_activation_width_sampled():
    # the GEMM workload's shape, [8192, 4096] activations from the activation workload's generator
    # times [4096, 4096] synthetic weights, checked on sampled rows against the oracle
    w_act = synth.WORKLOADS["activation_4096"]
    x = synth.make_x(w_act).reshape(w_act.tokens, w_act.head_dim)
    n, k = x.shape
    m = 4096
    w = synth.make_weights(m, k, seed=11, dtype="bf16")
    sg = synth.make_signs(w_act).reshape(k)
    s, xc, xa, wc, wb, y = _chain(x, w, sg, 128, 4)
    rows = np.random.default_rng(0).choice(n, size=48, replace=False)
    x64 = x[rows].double().numpy()
    act = oracle.rrs_quantize_act(x64, sg.numpy(), 128, s.double().numpy(), 4)
    parity.check_codes(xc.numpy()[rows], act, 4, sampled_from=n * k)
    parity.check_rel_f16(xa.numpy()[rows], act.scale, "activation scales")
    # the smoothing scales over all 8192 tokens, both sides (each is one token's rotated value)
    np.testing.assert_allclose(s.numpy(), oracle.rrs_smooth_scales(x.double().numpy(), sg.numpy(), 128), rtol=REL_S)
    # every weight code and scale of the 4096 x 4096 weights
    wq = oracle.rrs_quantize_weights(w.double().numpy(), sg.numpy(), 128, 4)
    wref = oracle.Quantized(codes=wq.codes[:, 0, :], packed=None, v=wq.v[:, 0, :], nu=None, scale=wq.scale[:, 0],
                            norms16=None, scales16=wq.scales16[:, 0])
    print("weight codes", parity.check_codes(wc.numpy(), wref, 4))
    parity.check_rel_f16(wb.numpy(), wref.scale, "weight scales")
    y_ref = oracle.rrs_gemm(oracle.unpack_nibbles(xc.numpy()[rows]), xa.numpy()[rows],
                            oracle.unpack_nibbles(wc.numpy()), wb.numpy(), s.double().numpy())
    _check_y(y.numpy()[rows], y_ref)
