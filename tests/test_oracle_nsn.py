"""Pins of the oracle's NSN variant (NSNQuant summary, "Normalize-Shift-Normalize (NSN)" and
"Hadamard transform").

Each pin checks nsn_quantize / nsn_dequantize against a property the definition fixes rather than
against a retyped formula: the two token norms, the zero block mean after the shift, exact
reconstruction when the quantizer is bypassed, invariance of the codes under a per-token scale,
the degenerate all-equal block, and the algebra the decode-score kernel folds the byproducts in
with.
"""
import numpy as np

import oracle

D, B = 64, 16


def _spec(seqs=2, tokens=2 * B, heads=3, bits=4, had=16):
    return oracle.Spec(seqs, tokens, heads, D, bits, "nsn_pchan", B, had)


def _input(seed, sp):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((sp.seqs * sp.tokens, sp.heads, D))
    x[..., 7] *= 25.0                                               # an outlier channel
    x += rng.standard_normal((1, sp.heads, D)) * 3.0                # a shared channel offset
    x *= rng.uniform(0.2, 5.0, size=(sp.seqs * sp.tokens, 1, 1))    # token norm swing
    signs = rng.choice(np.array([-1, 1], np.int8), size=(sp.heads, D)) if sp.hadamard else None
    return x, signs


def _directions(x, sp, signs):
    """u1, o, u2, u3 recomputed step by step from the returned scales (not from the oracle's code)."""
    y = oracle.rotate(x, signs, sp.hadamard) if sp.hadamard else x
    q = oracle.nsn_quantize(x, sp, signs)
    u1 = y / q.s1[..., None]
    u1b = u1.reshape(sp.seqs, sp.tokens // B, B, sp.heads, D)
    u2 = (u1b - u1b.mean(axis=2, keepdims=True)).reshape(u1.shape)
    u3 = u2 / q.s2[..., None]
    return q, u1, u2, u3


def test_token_norms_are_sqrt_d_and_the_block_mean_is_removed():
    sp = _spec()
    x, signs = _input(1, sp)
    q, u1, u2, u3 = _directions(x, sp, signs)
    np.testing.assert_allclose(np.linalg.norm(u1, axis=-1), np.sqrt(D), rtol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(u3, axis=-1), np.sqrt(D), rtol=1e-12)
    # the first scale is the input norm over sqrt(D) (the rotation is orthonormal)
    np.testing.assert_allclose(q.s1, np.linalg.norm(x, axis=-1) / np.sqrt(D), rtol=1e-12)
    # the shift leaves every channel of every block with mean zero
    blocks = u2.reshape(sp.seqs, sp.tokens // B, B, sp.heads, D)
    assert np.abs(blocks.sum(axis=2)).max() < 1e-12 * np.abs(blocks).max() * B
    # the codes are the rne quotients of u3 by the per-channel block scale, one of them at +-Q
    Q = oracle.qmax(sp.bits)
    c = q.codes.reshape(sp.seqs, sp.tokens // B, B, sp.heads, D)
    assert np.all(np.abs(c).max(axis=2) == Q)


def test_reconstruction_is_exact_without_the_quantizer():
    # replacing c * scale by u3 itself, the inverse steps give x back (fp64 round off only)
    sp = _spec()
    x, signs = _input(2, sp)
    q, u1, u2, u3 = _directions(x, sp, signs)
    back = oracle.inverse_rotate(u3, signs, sp.hadamard)
    off = np.repeat(q.offset.reshape(sp.seqs, sp.tokens // B, 1, sp.heads, D), B, axis=2).reshape(x.shape)
    xr = q.s1[..., None] * (q.s2[..., None] * back + off)
    np.testing.assert_allclose(xr, x, rtol=0, atol=1e-11 * np.abs(x).max())
    # and the stored dequantization is within the quantizer's half step of that
    xh = oracle.nsn_dequantize(q.packed, q.s1_16, q.s2_16, q.offset16, q.scales16, sp, signs)
    err = np.linalg.norm(xh - x) / np.linalg.norm(x)
    assert err < 0.2, err


def test_codes_ignore_a_per_token_scale():
    # the first normalization removes each token's scale: scaling tokens leaves every code alone
    sp = _spec(had=0)
    x, _ = _input(3, sp)
    lam = np.random.default_rng(4).uniform(0.01, 100.0, size=(x.shape[0], 1, 1))
    a = oracle.nsn_quantize(x, sp)
    b = oracle.nsn_quantize(x * lam, sp)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_allclose(b.s1, a.s1 * lam[..., 0], rtol=1e-12)


def test_a_block_of_equal_tokens():
    # every token equal: u2 = 0, so s2 = 0, codes 0, and x^ = s1 * offset = x (to fp16 rounding)
    sp = _spec(seqs=1, tokens=B, heads=1, had=16)
    rng = np.random.default_rng(5)
    row = rng.standard_normal(D)
    x = np.repeat(row[None, None, :], B, axis=0)
    signs = rng.choice(np.array([-1, 1], np.int8), size=(1, D))
    q = oracle.nsn_quantize(x, sp, signs)
    assert np.all(q.codes == 0) and np.all(q.s2 == 0.0)
    np.testing.assert_allclose(q.offset[0, 0], row / q.s1[0, 0], rtol=1e-12)
    xh = oracle.nsn_dequantize(q.packed, q.s1_16, np.zeros_like(q.s2_16), q.offset16, q.scales16, sp, signs)
    np.testing.assert_allclose(xh, x, rtol=2e-3, atol=2e-3 * np.abs(row).max())


def test_score_folds_the_byproducts():
    # q . x^_t = s1 s2 (R q) . (c * scale) + s1 (q . offset): the rotated-domain form the decode
    # score uses, against the plain dot product with the dequantized keys
    sp = _spec(seqs=2, tokens=3 * B, heads=2, had=32)
    x, signs = _input(6, sp)
    q = oracle.nsn_quantize(x, sp, signs)
    k_hat = oracle.nsn_dequantize(q.packed, q.s1_16, q.s2_16, q.offset16, q.scales16, sp, signs)
    qq = np.random.default_rng(7).standard_normal((sp.seqs, 4 * sp.heads, D))
    direct = oracle.score_decode(qq, k_hat, sp)
    G = 4
    folded = np.zeros_like(direct)
    s1 = q.s1_16.astype(np.float64).reshape(sp.seqs, sp.tokens, sp.heads)
    s2 = q.s2_16.astype(np.float64).reshape(sp.seqs, sp.tokens, sp.heads)
    c = oracle.unpack_nibbles(q.packed).astype(np.float64).reshape(sp.seqs, sp.tokens, sp.heads, D)
    sc = q.scales16.astype(np.float64).reshape(sp.seqs, sp.tokens // B, sp.heads, D)
    off = q.offset16.astype(np.float64).reshape(sp.seqs, sp.tokens // B, sp.heads, D)
    for s in range(sp.seqs):
        for hq in range(G * sp.heads):
            h = hq // G
            rqv = oracle.rotate(qq[s, hq][None, None, :], signs[h:h + 1], sp.hadamard)[0, 0]
            for t in range(sp.tokens):
                b = t // B
                folded[s, hq, t] = (s1[s, t, h] * s2[s, t, h] * np.dot(rqv, c[s, t, h] * sc[s, b, h])
                                    + s1[s, t, h] * np.dot(qq[s, hq], off[s, b, h]))
    np.testing.assert_allclose(folded, direct, rtol=1e-10, atol=1e-10 * np.abs(direct).max())


def near_constant_block(eps, b=B, d=D):
    """b tokens (8, 0, ...) except token 0, (8, eps, 0, ...): every token but the first differs
    from the block mean of the directions by about eps / b (norm), token 0 by (b - 1) eps / b."""
    x = np.zeros((b, 1, d))
    x[:, 0, 0] = 8.0
    x[0, 0, 1] = eps
    return x


def test_second_norm_threshold_position():
    # the second normalization counts as zero below ||u2|| = 2^-16 sqrt(D) = 2^-13 (D = 64); tokens
    # 1 .. B-1 have ||u2|| = eps / 16 up to O(eps^2), so eps = 15 2^-13 puts them just below it and
    # eps = 17 2^-13 just above
    sp = oracle.Spec(1, B, 1, D, 4, "nsn_pchan", B, 0)
    below = oracle.nsn_quantize(near_constant_block(15 * 2.0 ** -13), sp)
    assert np.all(below.s2[1:] == 0.0) and np.all(below.codes[1:] == 0)
    assert below.s2[0, 0] > 0.0
    above = oracle.nsn_quantize(near_constant_block(17 * 2.0 ** -13), sp)
    # s2 = ||u2|| / sqrt(D) = (eps / 16) / 8 to within O(eps^2)
    np.testing.assert_allclose(above.s2[1:, 0], 17 * 2.0 ** -13 / 16 / 8, rtol=1e-5)
    assert np.all(np.abs(above.codes[1:]).max(axis=-1) == 7)
    # below the threshold x^ = s1 * offset: the block mean of the directions, scaled back
    xh = oracle.nsn_dequantize(below.packed, below.s1_16, below.s2_16, below.offset16, below.scales16, sp)
    np.testing.assert_allclose(xh[1:, 0, 0], 8.0, rtol=1e-3)
