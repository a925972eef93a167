"""Inputs that lie exactly on the quantization grid (closed-form expected codes).

Every (token, head) vector is y = 2^p * 2^-e * k with integer codes k, sum_d k_d^2 = 4^e and
one entry equal to +-Q.  Then nu = 2^p, u = 2^-e k, scale = 2^-e, quotient = k, all exact in
binary floating point, so quantize must return k and dequantize must return x bit for bit.
With a rotation of size n in {16, 64} (1/sqrt n a power of two) the input is built as
x = sigma * H_n y / sqrt(n) using scipy's Sylvester Hadamard matrix, so the rotated vector is
exactly y again.  This module builds test inputs only; it does not call the oracle or the
HIP library.
"""
import numpy as np
import scipy.linalg

from oracle import Spec  # only the parameter record

# integer patterns with sum of squares 4^e and max |k| = Q
PATTERNS = {4: (3, [7, 3, 2, 1, 1]), 3: (2, [3, 2, 1, 1, 1]), 2: (1, [1, 1, 1, 1])}


def make(bits, mode, hadamard, head_dim=64, seqs=2, tokens=128, heads=2, seed=0):
    """Returns (spec, x float64 [N, H, D], signs int8 [H, D] or None, codes int8 [N, H, D])."""
    rng = np.random.default_rng(seed)
    D = head_dim
    B = D if "pchan" in mode else 0            # B tokens cover every channel with a +-Q
    spec = Spec(seqs, tokens, heads, D, bits, mode, B, hadamard)
    e, pat = PATTERNS[bits]
    N = seqs * tokens
    k = np.zeros((N, heads, D), dtype=np.int64)
    expo = np.zeros((N, heads))
    for r in range(N):
        t = r % tokens
        for h in range(heads):
            lead = (t + 3 * h) % D
            others = rng.choice(np.delete(np.arange(D), lead), size=len(pat) - 1, replace=False)
            pos = np.concatenate([[lead], others])
            k[r, h, pos] = np.array(pat) * rng.choice([-1, 1], size=len(pat))
    if mode == "pchan":
        # no norm separation: one exponent per (block, head) so each channel's max is Q 2^p
        for blk in range(N // B):
            expo[blk * B:(blk + 1) * B] = rng.integers(-3, 4, size=heads)
    else:
        expo[:] = rng.integers(-2, 4, size=(N, heads))
    if mode in ("naive", "pchan"):
        y = k * np.exp2(expo)[..., None]                    # scale = 2^p, quotient = k
    else:
        y = k * np.exp2(expo - e)[..., None]                # nu = 2^p, u = 2^-e k
    signs = None
    x = y
    if hadamard:
        n = hadamard
        signs = rng.choice(np.array([-1, 1], dtype=np.int8), size=(heads, D))
        H = scipy.linalg.hadamard(n).astype(np.float64)
        blocks = y.reshape(N, heads, D // n, n) @ H.T / np.sqrt(n)   # H symmetric
        x = blocks.reshape(N, heads, D) * signs[None]
    assert np.all(np.abs(x) < 60000)
    assert np.all(x.astype(np.float16).astype(np.float64) == x), "grid input not fp16-exact"
    return spec, x, signs, k.astype(np.int8)


def all_ties(had, seed=0, T=128, H=2, D=64, extra_max=0):
    """Every quotient an exact half-integer (or +-7): tokens are signed permutations of one
    multiset {7, half-integers} with the 7 in channel (t mod D), so all norms are equal and every
    per-token and per-channel max is 7 * 2^p.  extra_max > 0 turns that many of the half-integers
    into further 7s (the max then sits in several channels).  With a rotation of size 16 the
    input is sigma * H y / 4 of such a y (exact in fp16)."""
    rng = np.random.default_rng(seed)
    halves = rng.choice(np.arange(0.5, 7.0, 1.0), size=D - 1)
    halves[:extra_max] = 7.0
    y = np.zeros((T, H, D))
    for t in range(T):
        for h in range(H):
            vals = np.concatenate([[7.0], rng.permutation(halves)]) * rng.choice([-1, 1], size=D)
            pos = np.concatenate([[t % D], rng.permutation(np.delete(np.arange(D), t % D))])
            y[t, h, pos] = vals
    y *= 2.0 ** -2
    want = np.vectorize(lambda v: round(v))(y * 4.0).astype(np.int8)   # half-even, independent
    signs = None
    x = y
    if had:
        signs = rng.choice(np.array([-1, 1], np.int8), size=(H, D))
        Hm = scipy.linalg.hadamard(had).astype(np.float64)
        x = (y.reshape(T, H, D // had, had) @ Hm.T / np.sqrt(had)).reshape(T, H, D) * signs[None]
    assert np.all(x.astype(np.float16).astype(np.float64) == x)
    return x, signs, want


# Near-tie inputs: with a 16-point rotation, a block x = (a, b, c, 0, ...) of one token rotates to
# y_i = (a + H[i,1] b + H[i,2] c) / 4, and a tiny c (the smallest fp16 subnormal, 2^-24) moves every
# quotient off its tie by far less than an fp32 ulp of it.  Per bit width, (a, b) makes channel 1's
# quotient Q (a - b + c) / (a + b + c) a hair above a tie that half-to-even rounds down
# (2.5 at INT4 and INT3, 0.5 at 2 bits) and channel 3's, Q (a - b - c) / (a + b + c), a hair below
# it.  Decided on the fp64 quotient the two round apart; decided on its fp32 value both would
# become the tie itself.
NEAR_TIE_AB = {4: (9.5, 4.5), 3: (5.5, 0.5), 2: (24.0, 8.0)}
NEAR_TIE_C = 2.0 ** -24


def _hadamard_entry(i, j):
    return -1 if bin(i & j).count("1") % 2 else 1


def _rne(fr):
    """Round a Fraction half to even (exact)."""
    import fractions
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > fractions.Fraction(1, 2) or (rem == fractions.Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def near_ties(bits, per_channel, D=64, B=64):
    """x float64 [B, 1, D] (one head, one sequence of B tokens), signs int8 [1, D] (all +1) and the
    expected codes int8 [B, 1, D], derived in exact rational arithmetic (no oracle, no floating
    point).  Per-token modes: token 2k + s is (+-a, +-b, c) (s picks the sign of b, k the overall
    sign) in the first 16-channel block and zero elsewhere.  Per-channel modes: the same four
    tokens 0..3 and zero tokens after them, so channel i's block max is the larger of its two
    magnitudes (a + b +- c)."""
    import fractions
    F = fractions.Fraction
    Q = (1 << (bits - 1)) - 1
    a, b = NEAR_TIE_AB[bits]
    c = NEAR_TIE_C
    T = B
    x = np.zeros((T, 1, D))
    rows = 4 if per_channel else T
    for t in range(rows):
        sb = 1.0 if (t % 2 == 0) else -1.0
        sg = 1.0 if ((t // 2) % 2 == 0) else -1.0
        x[t, 0, :3] = sg * np.array([a, sb * b, c])
    assert np.all(x.astype(np.float16).astype(np.float64) == x)
    # exact rotation of every token (the 1/4 cancels in every quotient; kept for clarity)
    y = [[sum(_hadamard_entry(i % 16, j % 16) * F(x[t, 0, j]) for j in range(16 * (i // 16), 16 * (i // 16) + 16)) / 4
          for i in range(D)] for t in range(T)]
    want = np.zeros((T, 1, D), dtype=np.int8)
    for t in range(T):
        for i in range(D):
            m = max(abs(y[s][i]) for s in range(T)) if per_channel else max(abs(v) for v in y[t])
            want[t, 0, i] = 0 if m == 0 else max(-Q, min(Q, _rne(Q * y[t][i] / m)))
    return x, np.ones((1, D), dtype=np.int8), want
