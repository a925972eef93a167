"""GPU parity of the NSN variant (kvq_quantize_nsn, kvq_dequantize_nsn, kvq_score_decode_nsn)
against the fp64 oracle (oracle.nsn_quantize / nsn_dequantize / score_decode) on the same seeded
inputs, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from activation_quantization_amd import kvq
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _input(seed, S, T, H, D, dtype, had):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((S * T, H, D)).astype(np.float32)
    x[..., 3] *= 30.0                                                   # an outlier channel
    x += rng.standard_normal((1, H, D)).astype(np.float32) * 2.0        # a shared channel offset
    x *= rng.uniform(0.3, 4.0, size=(S * T, 1, 1)).astype(np.float32)   # token norm swing
    signs = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=(H, D))) if had else None
    return torch.from_numpy(x).to(dtype), signs


def _spec(d):
    return oracle.Spec(d.seqs, d.tokens_per_seq, d.heads, d.head_dim, d.bits, "nsn_pchan", d.block_tokens, d.hadamard)


def _check_offsets(gpu16, ref64):
    # stored offsets are fp16 roundings of the fp64 mean (original domain): 1e-3 of the value or of
    # the rms of its block's offset vector, whichever is larger
    g = np.asarray(gpu16, dtype=np.float64)
    r = np.asarray(ref64, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    bad = np.abs(g - r) > 1e-3 * np.maximum(np.abs(r), rms)
    assert not np.any(bad), f"offsets: {int(bad.sum())} outside tolerance"


def _run(d, x, signs, q_heads=None):
    sg = None if signs is None else signs.to(DEV)
    out = kvq.quantize_nsn(d, x.to(DEV), sg)
    torch.cuda.synchronize()
    codes, s1, s2, offsets, scales = out
    sp = _spec(d)
    sg_np = None if signs is None else signs.numpy()
    ref = oracle.nsn_quantize(x.double().numpy(), sp, sg_np)
    tc, ts1, tsc = kvq.token_major(d, codes, s1, scales)
    _, ts2, toff = kvq.token_major(d, None, s2, offsets)
    gc, g1, g2, goff, gsc = (t.cpu().numpy() for t in (tc, ts1, ts2, toff, tsc))
    stats = parity.check_codes(gc, ref, d.bits)
    parity.check_rel_f16(g1, ref.s1, "s1")
    parity.check_rel_f16(g2, ref.s2, "s2")
    parity.check_rel_f16(gsc, ref.scale, "scales")
    _check_offsets(goff, ref.offset)
    # dequantize from the GPU's own stored values
    ref_dq = oracle.nsn_dequantize(gc, g1, g2, goff, gsc, sp, sg_np)
    y = kvq.dequantize_nsn(d, codes, s1, s2, offsets, scales, sg, torch.float32)
    torch.cuda.synchronize()
    parity.check_dequant(y.cpu().numpy(), ref_dq)
    y2 = kvq.dequantize_nsn(d, codes, s1, s2, offsets, scales, sg, d.dtype)
    torch.cuda.synchronize()
    parity.check_dequant_lowp(y2.cpu(), ref_dq, "f16" if d.dtype == torch.float16 else "bf16")
    if q_heads:
        q = torch.from_numpy(np.random.default_rng(9).standard_normal((d.seqs, q_heads, d.head_dim))
                             .astype(np.float32)).half()
        sc = kvq.score_decode_nsn(d, q.to(DEV), codes, s1, s2, offsets, scales, sg)
        torch.cuda.synchronize()
        parity.check_scores(sc.cpu().numpy(), oracle.score_decode(q.double().numpy(), ref_dq, sp),
                            q.double().numpy(), ref_dq, sp)
    return stats, ref


@pytest.mark.parametrize("D,B,had", [(128, 128, 128), (128, 64, 0), (64, 64, 16), (64, 256, 64), (128, 128, 32)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_nsn_parity(D, B, had, dtype):
    S, T, H = 2, 2 * B, 3
    x, signs = _input(D + B + had, S, T, H, D, dtype, had)
    d = kvq.Desc(S, T, H, D, 4, "nsn_pchan", B, had, dtype)
    stats, _ = _run(d, x, signs, q_heads=4 * H)
    print(stats)


@pytest.mark.parametrize("bits", [3, 2])
def test_nsn_bits(bits):
    S, T, H, D, B = 2, 256, 2, 128, 128
    x, signs = _input(bits, S, T, H, D, torch.float16, 128)
    d = kvq.Desc(S, T, H, D, bits, "nsn_pchan", B, 128, torch.float16)
    _run(d, x, signs, q_heads=2 * H)


def test_nsn_degenerate_blocks():
    # a block of identical tokens (s2 = 0, codes 0) next to an ordinary block, and a zero token
    S, T, H, D, B = 1, 128, 1, 128, 64
    x, signs = _input(11, S, T, H, D, torch.float16, 128)
    x[:B] = x[0:1]
    x[B + 5] = 0
    d = kvq.Desc(S, T, H, D, 4, "nsn_pchan", B, 128, torch.float16)
    _, ref = _run(d, x, signs, q_heads=4)
    assert np.all(ref.codes[:B] == 0) and np.all(ref.s2[:B] == 0)


def test_plain_entry_points_refuse_nsn():
    d = kvq.Desc(1, 128, 1, 128, 4, "nsn_pchan", 128, 0, torch.float16)
    x = torch.zeros((128, 1, 128), dtype=torch.float16, device=DEV)
    with pytest.raises(kvq.KvqError):
        kvq.quantize(d, x, None, out=kvq.alloc_outputs(kvq.Desc(1, 128, 1, 128, 4, "pchan", 128, 0), DEV))


@pytest.mark.parametrize("factor", [15, 17])
def test_second_norm_threshold(factor):
    # tokens 1 .. 63 of a 64-token block differ from the block mean of the directions by
    # ||u2|| = eps / 64 (to O(eps^2)); eps = 15 or 17 2^-11 puts that just below or just above the
    # zero threshold 2^-16 sqrt(64): s2 = 0 and codes 0 below it, s2 = ||u2|| / 8 above it
    from tests.test_oracle_nsn import near_constant_block
    x64 = near_constant_block(factor * 2.0 ** -11, b=64, d=64)
    d = kvq.Desc(1, 64, 1, 64, 4, "nsn_pchan", 64, 0, torch.float16)
    x = torch.from_numpy(x64).half()
    assert torch.equal(x.double(), torch.from_numpy(x64))
    _run(d, x, None)
    codes, s1, s2, offsets, scales = kvq.quantize_nsn(d, x.to(DEV), None)
    g2 = s2.cpu().numpy().reshape(64).astype(np.float64)
    c = oracle.unpack_nibbles(codes.cpu().numpy()).reshape(64, 64)
    if factor == 15:
        assert np.all(g2[1:] == 0.0) and not np.any(c[1:])
    else:
        np.testing.assert_allclose(g2[1:], factor * 2.0 ** -11 / 64 / 8, rtol=1e-3)
        assert np.all(np.abs(c[1:]).max(axis=-1) == 7)
