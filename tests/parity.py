"""Comparison of HIP-path outputs with the fp64 oracle, to the stated tolerances.

  codes   equal, except +-1 where the oracle's quotient |v| lies within TIE_BAND of a
          half-integer (a rounding tie decided the other way by fp32 rounding noise), on at
          most 1e-6 of the elements checked
  norms / scales   |gpu - ref| <= 1e-3 |ref| (one fp16 ulp), or one subnormal fp16 ulp
  dequantized      |gpu - ref| <= 1e-3 max(|ref|, rms of the reference vector)
  scores           |gpu - ref| <= 2e-3 max(|ref|, ||q|| ||k^|| / sqrt(D))
"""
from __future__ import annotations

import math

import numpy as np

import oracle

TIE_BAND = 2.0 ** -18
CODE_RATE = 1e-6
REL_PARAM = 1e-3
REL_DEQ = 1e-3
REL_SCORE = 2e-3
F16_SUBNORMAL_ULP = 2.0 ** -24


def tie_budget(n_checked: int, sampled_from: int | None = None) -> int:
    """Allowed tie flips: 1e-6 of the elements checked.  A sample drawn from a tensor of
    >= 1e6 elements may hold one flip (the rate applies to the whole tensor)."""
    b = int(math.floor(CODE_RATE * n_checked))
    if sampled_from is not None and sampled_from >= 1_000_000:
        b = max(b, 1)
    return b


def check_codes(gpu_packed: np.ndarray, ref: oracle.Quantized, bits: int, sampled_from=None) -> dict:
    Q = oracle.qmax(bits)
    g = oracle.unpack_nibbles(np.asarray(gpu_packed)).astype(np.int16)
    r = ref.codes.astype(np.int16)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert g.min() >= -Q and g.max() <= Q, "GPU code outside [-Q, Q]"
    diff = g != r
    n_diff = int(diff.sum())
    if n_diff:
        d = np.abs(g[diff] - r[diff])
        av = np.abs(ref.v[diff])
        dist = np.abs(av - np.floor(av) - 0.5)
        assert np.all(d == 1), f"code differs by more than 1 at {np.argwhere(diff)[:5].tolist()}"
        assert np.all(dist < TIE_BAND), (
            f"{int(np.sum(dist >= TIE_BAND))} code mismatches away from a rounding tie, "
            f"worst distance {dist.max():.3g}, first at {np.argwhere(diff)[:3].tolist()}")
    budget = tie_budget(g.size, sampled_from)
    assert n_diff <= budget, f"{n_diff} tie flips > budget {budget} of {g.size} codes"
    return {"codes": g.size, "tie_flips": n_diff}


def check_rel_f16(gpu_f16: np.ndarray, ref64: np.ndarray, what: str):
    g = np.asarray(gpu_f16).astype(np.float64)
    r = np.asarray(ref64, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    err = np.abs(g - r)
    ok = (err <= REL_PARAM * np.abs(r)) | (err <= F16_SUBNORMAL_ULP)
    assert np.all(ok), f"{what}: {int((~ok).sum())} outside 1e-3 relative, worst rel {np.max(err / np.maximum(np.abs(r), 1e-30)):.3g}"


def check_dequant(gpu: np.ndarray, ref: np.ndarray):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    tol = REL_DEQ * np.maximum(np.abs(r), rms)
    bad = np.abs(g - r) > tol
    assert not np.any(bad), f"dequant: {int(bad.sum())} outside tolerance, first {np.argwhere(bad)[:3].tolist()}"


def check_dequant_lowp(gpu_lowp, ref: np.ndarray, dtype_name: str):
    """Output in fp16/bf16: each value equals the reference rounded to that dtype within one
    ulp, or lies within the fp32 tolerance above (near-zero values after the inverse rotation
    carry fp32 evaluation error larger than one low-precision ulp at their own magnitude)."""
    import torch
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype_name]
    r64 = np.asarray(ref, dtype=np.float64)
    r = torch.from_numpy(r64).to(tdt)
    g = gpu_lowp if isinstance(gpu_lowp, torch.Tensor) else torch.from_numpy(gpu_lowp)
    gi = g.view(torch.int16).to(torch.int32)
    ri = r.view(torch.int16).to(torch.int32)

    def ordered(v):  # sign-magnitude bits -> monotone integers
        return torch.where(v < 0, -(v & 0x7fff), v)
    ulps = (ordered(gi) - ordered(ri)).abs().numpy()
    rms = np.sqrt(np.mean(r64 * r64, axis=-1, keepdims=True))
    err = np.abs(g.double().numpy() - r64)
    ok = (ulps <= 1) | (err <= REL_DEQ * np.maximum(np.abs(r64), rms))
    assert np.all(ok), f"{dtype_name} dequant: {int((~ok).sum())} values off by {int(ulps[~ok].max())} ulp"


def check_scores(gpu: np.ndarray, ref: np.ndarray, q: np.ndarray, k_hat: np.ndarray, spec: oracle.Spec):
    """gpu/ref [S, Hq, T]; q [S, Hq, D]; k_hat [S*T, H, D]."""
    S, Hq, T = ref.shape
    G = Hq // spec.heads
    qn = np.linalg.norm(np.asarray(q, np.float64), axis=-1)                       # [S, Hq]
    kn = np.linalg.norm(k_hat, axis=-1).reshape(S, T, spec.heads)                 # [S, T, H]
    scale = qn[:, :, None] * np.repeat(kn, G, axis=2).transpose(0, 2, 1) / math.sqrt(spec.head_dim)
    tol = REL_SCORE * np.maximum(np.abs(ref), scale)
    err = np.abs(np.asarray(gpu, np.float64) - ref)
    bad = err > tol
    ratio = np.divide(err, tol, out=np.where(err > 0, np.inf, 0.0), where=tol > 0)   # 0 / 0: exact zero
    assert not np.any(bad), f"scores: {int(bad.sum())} outside tolerance, worst {np.max(ratio):.3g}x"
    return float(np.max(ratio))


REL_ATTN = 2e-3


def check_attention(gpu: np.ndarray, ref: np.ndarray):
    """gpu/ref [S, Hq, D]: |gpu - ref| <= 2e-3 max(|ref|, rms of the reference vector).  The output
    is a convex combination of value vectors, so its own rms is the natural magnitude floor."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    tol = REL_ATTN * np.maximum(np.abs(r), rms)
    err = np.abs(g - r)
    bad = err > tol
    assert not np.any(bad), f"attention: {int(bad.sum())} outside tolerance, worst {np.max(err / tol):.3g}x"
    return float(np.max(err / tol))
