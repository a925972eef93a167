"""fp64 CPU oracle for the transform-and-quantize path (KV cache / activations).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this module.  It shares no code, table or constant with the HIP
library and imports nothing from it; both sides only read the same seeded inputs.

Every step is the plain definition, in float64, in the order the pages give it:

  rotation   y = (1/sqrt(n)) H_n diag(sigma) x per n-channel block, H_n the Sylvester
             Hadamard matrix in natural order, sigma in {-1,+1}           (C1)
  norm sep.  nu = ||y||_2, u = y / nu (NSEP modes only)                    (C2)
  scale      per token: max_d |u| / Q ; per channel: max over a block of B
             tokens of |u_td| / Q ; Q = 2^(b-1) - 1                        (C3)
  codes      c = clamp(rne(u / scale), -Q, Q)                              (C4)
  packing    two's-complement nibbles, even channel in the low nibble      (C5)
  dequant    y^ = c * S16 * N16, then the inverse rotation                 (C6)
  score      s[q, t] = sum_d q_d * k^_td, query head hq reads KV head hq // G (C7)

Sources (page title, section):
  * norm-separation post ("nsep+pchan" for INT4/INT3 KV caches): "the fix", its four-line
    PyTorch snippet (L2 norm, unit direction, absmax/7, round and clamp to +-7); "root
    cause" (per-row absmax, outlier channels); the ".norm() pitfall" (an L2 norm, not
    L_{-1}).
  * Rotated Runtime Smooth analysis (ICLR): "problem definition" (alpha = max|X|/(2^(N-1)-1)),
    "master equation" and "term-by-term" (R = (1/sqrt K)[+-1], R R^T = I, s_j = column max),
    Figure 2 (Y = (XR)(R^-1 W^T) = X W^T), "experimental design" (RTN, group size 128).
  * NSNQuant summary: "Hadamard transform" (randomized Hadamard), "implementation details"
    (scores computed with the stored byproducts folded in, dequantization kernel).
  * Activation-guided compensation abstract: random signs before the Hadamard rotation.

Readings where the pages are silent or garbled (each also listed in the design doc):
  R1 rotation is orthonormal (1/sqrt n); signs first, then H; natural Sylvester order;
     one sign vector per head shared by all tokens; block k of a wide row uses
     sigma[k n:(k+1) n].
  R2 "per-channel" = max over the tokens of one B-token block of one sequence; the
     snippet's amax over the last dim is the per-token NSEP mode.
  R3 codes use the unrounded scale and norm; stored values are fp16(nu), fp16(scale).
  R4 rounding is half-to-even on the exact (fp64) quotient, as the snippet's .round() does:
     c = clamp(rne(u / scale), -Q, Q).
  R5 nu = 0 or scale = 0 give codes 0 and stored 0.
  R6 the decode score is the plain dot product q . k^ (no 1/sqrt d, no softmax), with
     k^ the fp64 dequantized key before any output rounding.
"""
from __future__ import annotations

import dataclasses
from fractions import Fraction

import numpy as np

MODES = ("naive", "nsep", "pchan", "nsep_pchan")
NSN_MODE = "nsn_pchan"        # NSN before the per-channel quantizer (its own entry points)


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and method parameters; x is [seqs * tokens, heads, head_dim]."""
    seqs: int
    tokens: int
    heads: int
    head_dim: int
    bits: int
    mode: str
    block_tokens: int = 0     # per-channel token block B (pchan modes)
    hadamard: int = 0         # 0 = no rotation, else the Hadamard block size n

    @property
    def nsep(self) -> bool:
        return self.mode in ("nsep", "nsep_pchan")

    @property
    def per_channel(self) -> bool:
        return self.mode in ("pchan", "nsep_pchan", "nsn_pchan")


def qmax(bits: int) -> int:
    """Q = 2^(b-1) - 1: +-7 at INT4 (the snippet's clamp), +-3 at INT3, +-1 at 2 bits."""
    return (1 << (bits - 1)) - 1


# ----------------------------------------------------------------------------- rotation
def hadamard_matrix(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix in natural order: H[i, j] = (-1)^popcount(i & j)."""
    i = np.arange(n, dtype=np.int64)
    a = i[:, None] & i[None, :]
    parity = np.zeros_like(a)
    while np.any(a):
        parity ^= a & 1
        a >>= 1
    return np.where(parity == 1, -1.0, 1.0)


def rotate(x: np.ndarray, signs: np.ndarray, n: int) -> np.ndarray:
    """y = (1/sqrt n) H_n (sigma * x) on every n-channel block of every [.., heads, D] row.

    x: float64 [N, heads, D]; signs: [heads, D] of +-1.
    """
    N, Hh, D = x.shape
    xs = x * signs.astype(np.float64)[None, :, :]
    blocks = xs.reshape(N, Hh, D // n, n)
    y = blocks @ hadamard_matrix(n).T / np.sqrt(n)
    return y.reshape(N, Hh, D)


def inverse_rotate(y: np.ndarray, signs: np.ndarray, n: int) -> np.ndarray:
    """x = sigma * (1/sqrt n) H_n^T y: the transpose of `rotate` (R^-1 = R^T)."""
    N, Hh, D = y.shape
    blocks = y.reshape(N, Hh, D // n, n)
    x = (blocks @ hadamard_matrix(n) / np.sqrt(n)).reshape(N, Hh, D)
    return x * signs.astype(np.float64)[None, :, :]


# ----------------------------------------------------------------------------- rounding
# The code is rne of the exact quotient (the snippet's .round() on the exact value).  fp64 decides
# it everywhere except within TIE_CHECK of a half-integer, where the few roundings of the fp64
# steps could put the value on either side of the tie: there the decision is taken exactly, in
# rational arithmetic, from the squared quotient (norms enter squared, so no square root is needed).
TIE_CHECK = 2.0 ** -36


def _rne_from_square(sign: int, q2: Fraction) -> int:
    """rne(v) for v = sign * sqrt(q2), exactly: k = floor(|v|), then |v| against k + 1/2."""
    k = 0
    while (k + 1) * (k + 1) <= q2:
        k += 1
    half2 = Fraction(2 * k + 1, 2) ** 2
    if q2 > half2 or (q2 == half2 and k % 2 == 1):
        k += 1
    return sign * k


def _near_tie(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    return np.abs(a - np.floor(a) - 0.5) < TIE_CHECK


def _exact_rotation(x_row: np.ndarray, signs_row, n: int) -> list:
    """Y = H_n diag(sigma) x of one vector as exact Fractions, without the 1/sqrt(n) factor (it
    cancels in every quotient); the identity when n == 0."""
    xs = [Fraction(float(e)) * (int(signs_row[j]) if signs_row is not None else 1) for j, e in enumerate(x_row)]
    if not n:
        return xs
    out = []
    for c in range(len(xs)):
        b = (c // n) * n
        out.append(sum(xs[b + j] if bin((c % n) & j).count("1") % 2 == 0 else -xs[b + j] for j in range(n)))
    return out


def _round_codes(v: np.ndarray, Q: int, exact_square) -> np.ndarray:
    """c = clamp(rne(v), -Q, Q); near a tie the exact quotient decides: exact_square(index) returns
    (sign, v^2) as an int and a Fraction."""
    c = np.rint(v)
    for idx in zip(*np.nonzero(_near_tie(v) & (v != 0.0))):
        c[idx] = _rne_from_square(*exact_square(idx))
    return np.clip(c, -Q, Q).astype(np.int8)


# ----------------------------------------------------------------------------- quantize
@dataclasses.dataclass
class Quantized:
    codes: np.ndarray      # int8 [N, heads, D] in [-Q, Q]
    packed: np.ndarray     # uint8 [N, heads, D/2]
    v: np.ndarray          # float64 quotient u / scale before rounding [N, heads, D]
    nu: np.ndarray | None  # float64 norms [N, heads] (NSEP modes)
    scale: np.ndarray      # float64 scales: [N, heads] or [seqs * T/B, heads, D]
    norms16: np.ndarray | None   # float16 stored norms
    scales16: np.ndarray         # float16 stored scales


def quantize(x: np.ndarray, spec: Spec, signs: np.ndarray | None = None) -> Quantized:
    """Quantize x ([N, heads, D], any float dtype, widened exactly to float64)."""
    x = np.asarray(x, dtype=np.float64)
    N, Hh, D = x.shape
    assert N == spec.seqs * spec.tokens and Hh == spec.heads and D == spec.head_dim
    Q = qmax(spec.bits)

    # C1: optional randomized Hadamard rotation
    y = rotate(x, signs, spec.hadamard) if spec.hadamard else x.copy()

    # C2: norm separation -> unit direction
    nu = None
    if spec.nsep:
        nu = np.sqrt(np.sum(y * y, axis=-1))
        safe = np.where(nu > 0.0, nu, 1.0)
        u = np.where(nu[..., None] > 0.0, y / safe[..., None], 0.0)
    else:
        u = y

    # C3: the scale, per token or per channel over a block of B tokens
    if spec.per_channel:
        B = spec.block_tokens
        nb = spec.tokens // B
        ub = np.abs(u).reshape(spec.seqs, nb, B, Hh, D)
        scale = (ub.max(axis=2) / Q).reshape(spec.seqs * nb, Hh, D)
        scale_full = np.repeat(scale.reshape(spec.seqs, nb, 1, Hh, D), B, axis=2).reshape(N, Hh, D)
    else:
        scale = np.abs(u).max(axis=-1) / Q
        scale_full = np.broadcast_to(scale[..., None], u.shape)

    # C4: quotient, round half to even, clamp
    safe = np.where(scale_full > 0.0, scale_full, 1.0)
    v = np.where(scale_full > 0.0, u / safe, 0.0)

    # the exact quotient near a tie: u / scale = Q u_c / max|u| over the scale's group, where the
    # rotation's 1/sqrt(n) cancels and, per token, so does the norm; per channel with NSEP,
    # (u_tc)^2 = Y_tc^2 / ||Y_t||^2
    rot, nrm2, colmax = {}, {}, {}

    def Y(r, h):
        if (r, h) not in rot:
            rot[r, h] = _exact_rotation(x[r, h], None if signs is None else signs[h], spec.hadamard)
        return rot[r, h]

    def u2(r, h, d):                       # the squared direction entry (up to the common 1/n)
        if not spec.nsep:
            return Y(r, h)[d] ** 2
        if (r, h) not in nrm2:
            nrm2[r, h] = sum(e * e for e in Y(r, h))
        return Y(r, h)[d] ** 2 / nrm2[r, h] if nrm2[r, h] else Fraction(0)

    def exact_square(idx):
        r, h, d = (int(i) for i in idx)
        if spec.per_channel:
            first = (r // spec.block_tokens) * spec.block_tokens
            if (first, h, d) not in colmax:
                colmax[first, h, d] = max(u2(t, h, d) for t in range(first, first + spec.block_tokens))
            num, m2 = u2(r, h, d), colmax[first, h, d]
        else:
            if (r, h) not in colmax:
                colmax[r, h] = max(e * e for e in Y(r, h))
            num, m2 = Y(r, h)[d] ** 2, colmax[r, h]
        return (1 if Y(r, h)[d] > 0 else -1), Fraction(Q * Q) * num / m2

    c = _round_codes(v, Q, exact_square)

    return Quantized(codes=c, packed=pack_nibbles(c), v=v, nu=nu, scale=scale,
                     norms16=None if nu is None else nu.astype(np.float16),
                     scales16=scale.astype(np.float16))


# ----------------------------------------------------------------------------- packing
def pack_nibbles(c: np.ndarray) -> np.ndarray:
    """Two 4-bit two's-complement codes per byte; channel 2i low nibble, 2i+1 high."""
    c = c.astype(np.int16)
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles; nibbles are sign-extended."""
    b = b.astype(np.int16)
    nib = np.stack([b & 0xF, b >> 4], axis=-1).reshape(*b.shape[:-1], b.shape[-1] * 2)
    return np.where(nib >= 8, nib - 16, nib).astype(np.int8)


# ----------------------------------------------------------------------------- dequantize
def expand_scales(scales16: np.ndarray, spec: Spec) -> np.ndarray:
    """Stored scales broadcast to every element [N, heads, D] as float64."""
    s = np.asarray(scales16).astype(np.float64)
    N, Hh, D = spec.seqs * spec.tokens, spec.heads, spec.head_dim
    if spec.per_channel:
        B = spec.block_tokens
        nb = spec.tokens // B
        return np.repeat(s.reshape(spec.seqs, nb, 1, Hh, D), B, axis=2).reshape(N, Hh, D)
    return np.broadcast_to(s.reshape(N, Hh, 1), (N, Hh, D))


def dequantize(packed: np.ndarray, norms16, scales16, spec: Spec,
               signs: np.ndarray | None = None) -> np.ndarray:
    """x^ in float64: codes * scale (* norm), then the inverse rotation.

    The inputs are the stored (fp16) norms and scales, exactly widened.
    """
    c = unpack_nibbles(np.asarray(packed)).astype(np.float64)
    y = c * expand_scales(scales16, spec)
    if spec.nsep:
        y = y * np.asarray(norms16).astype(np.float64)[..., None]
    return inverse_rotate(y, signs, spec.hadamard) if spec.hadamard else y


# ----------------------------------------------------------------------------- decode score
def score_decode(q: np.ndarray, k_hat: np.ndarray, spec: Spec) -> np.ndarray:
    """scores[s, hq, t] = sum_d q[s, hq, d] * k^[s*T + t, hq // G, d] in float64.

    q: [seqs, q_heads, D]; k_hat: dequantized keys [seqs*T, heads, D] (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    S, Hq, D = q.shape
    G = Hq // spec.heads
    kh = k_hat.reshape(S, spec.tokens, spec.heads, D)
    out = np.empty((S, Hq, spec.tokens))
    for hq in range(Hq):
        out[:, hq, :] = np.einsum("sd,std->st", q[:, hq, :], kh[:, :, hq // G, :])
    return out


# ----------------------------------------------------------------------------- decode attention
def attention_decode(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, spec: Spec) -> np.ndarray:
    """One decode step of attention over the whole cache, in float64 (the step after the decode
    score: NSNQuant summary, "implementation details" and "latency"; the norm-separation post,
    "longer contexts get worse", on error accumulating in attention as the cache grows).

    out[s, hq, :] = sum_t p[t] v^[s*T + t, hq // G, :],  p = softmax_t(q . k^_t / sqrt(D)),
    with plain scores q . k^ as in score_decode.  q: [seqs, q_heads, D]; k_hat, v_hat: the
    dequantized caches [seqs*T, heads, D].
    """
    sc = score_decode(q, k_hat, spec) / np.sqrt(spec.head_dim)          # [S, Hq, T]
    sc = sc - sc.max(axis=-1, keepdims=True)                             # exp() is then <= 1
    p = np.exp(sc)
    p /= p.sum(axis=-1, keepdims=True)
    S, Hq, T = p.shape
    G = Hq // spec.heads
    vh = np.asarray(v_hat, dtype=np.float64).reshape(S, T, spec.heads, spec.head_dim)
    out = np.empty((S, Hq, spec.head_dim))
    for hq in range(Hq):
        out[:, hq, :] = np.einsum("st,std->sd", p[:, hq, :], vh[:, :, hq // G, :])
    return out


# ----------------------------------------------------------------------------- NSN variant
@dataclasses.dataclass
class NsnQuantized:
    codes: np.ndarray        # int8 [N, heads, D]
    packed: np.ndarray       # uint8 [N, heads, D/2]
    v: np.ndarray            # float64 quotient before rounding
    s1: np.ndarray           # float64 [N, heads]: first token scale, ||x|| / sqrt(D)
    s2: np.ndarray           # float64 [N, heads]: second token scale, ||u1 - o|| / sqrt(D)
    offset: np.ndarray       # float64 [seqs * T/B, heads, D]: the block's channel mean, original domain
    scale: np.ndarray        # float64 [seqs * T/B, heads, D]: per-channel absmax / Q of u3
    s1_16: np.ndarray
    s2_16: np.ndarray
    offset16: np.ndarray
    scales16: np.ndarray


def nsn_quantize(x: np.ndarray, spec: Spec, signs: np.ndarray | None = None) -> NsnQuantized:
    """Normalize-Shift-Normalize before the per-channel scalar quantizer (NSNQuant summary,
    "Normalize-Shift-Normalize (NSN)": token norms to sqrt(d), subtract the channel means, token
    norms to sqrt(d) again, keeping s1, o, s2 to reconstruct; "Hadamard transform": combined with a
    randomized Hadamard rotation).

    Per (token, head): y = R x (C1), s1 = ||y|| / sqrt(D), u1 = y / s1.  Per (sequence, B-token
    block, head): o = the mean of u1 over the block's tokens.  Per token: u2 = u1 - o,
    s2 = ||u2|| / sqrt(D), u3 = u2 / s2.  Then per-channel absmax / Q of u3 over the block and
    c = rne(u3 / scale) as in quantize().  The rotation is orthonormal and linear, so it
    commutes with both normalizations and with the mean; the stored offset is the mean in the
    original domain, R^T o.  s1 = 0 or s2 = 0 give zero directions (and codes 0); s2 counts as 0
    when ||u2|| < 2^-16 sqrt(D) (reading: a token equal to its block's mean up to round-off).
    """
    x = np.asarray(x, dtype=np.float64)
    N, Hh, D = x.shape
    assert spec.mode == "nsn_pchan" and N == spec.seqs * spec.tokens
    Q = qmax(spec.bits)
    B = spec.block_tokens
    nb = spec.tokens // B
    y = rotate(x, signs, spec.hadamard) if spec.hadamard else x.copy()

    def unit(v):                       # scale to norm sqrt(D); returns (direction, scale)
        sc = np.sqrt(np.sum(v * v, axis=-1)) / np.sqrt(D)
        safe = np.where(sc > 0.0, sc, 1.0)
        return np.where(sc[..., None] > 0.0, v / safe[..., None], 0.0), sc

    u1, s1 = unit(y)
    o = u1.reshape(spec.seqs, nb, B, Hh, D).mean(axis=2)                                 # [S, nb, H, D]
    u2 = u1 - np.repeat(o[:, :, None], B, axis=2).reshape(N, Hh, D)
    # a token equal to its block's mean up to round-off (||u2|| under 2^-16 of ||u1|| = sqrt(D))
    # has no second direction: s2 = 0, codes 0 (else round-off noise would fill the codes)
    u2 = np.where((np.sqrt(np.sum(u2 * u2, axis=-1)) < 2.0 ** -16 * np.sqrt(D))[..., None], 0.0, u2)
    u3, s2 = unit(u2)
    amax = np.abs(u3).reshape(spec.seqs, nb, B, Hh, D).max(axis=2)
    scale = (amax / Q).reshape(spec.seqs * nb, Hh, D)
    scale_full = np.repeat(scale.reshape(spec.seqs, nb, 1, Hh, D), B, axis=2).reshape(N, Hh, D)
    safe = np.where(scale_full > 0.0, scale_full, 1.0)
    v = np.where(scale_full > 0.0, u3 / safe, 0.0)
    # rne of the fp64 quotient: the shift subtracts a mean of directions scaled by irrational norms,
    # so there is no rational form of the exact quotient to decide near-ties with; the fp64 value
    # is within a few ulp of it
    c = np.clip(np.rint(v), -Q, Q).astype(np.int8)
    o = o.reshape(spec.seqs * nb, Hh, D)
    offset = inverse_rotate(o, signs, spec.hadamard) if spec.hadamard else o
    return NsnQuantized(codes=c, packed=pack_nibbles(c), v=v, s1=s1, s2=s2, offset=offset, scale=scale,
                        s1_16=s1.astype(np.float16), s2_16=s2.astype(np.float16),
                        offset16=offset.astype(np.float16), scales16=scale.astype(np.float16))


def nsn_dequantize(packed: np.ndarray, s1_16, s2_16, offset16, scales16, spec: Spec,
                   signs: np.ndarray | None = None) -> np.ndarray:
    """x^ = s1 (s2 R^T (c * scale) + offset) in float64 from the stored fp16 byproducts (the
    inverse of each NSN step, in reverse order)."""
    c = unpack_nibbles(np.asarray(packed)).astype(np.float64)
    u3 = c * expand_scales(scales16, spec)
    back = inverse_rotate(u3, signs, spec.hadamard) if spec.hadamard else u3
    off = expand_scales(offset16, spec)                 # the same per-block broadcast as the scales
    s1 = np.asarray(s1_16).astype(np.float64)[..., None]
    s2 = np.asarray(s2_16).astype(np.float64)[..., None]
    return s1 * (s2 * back + off)


# ----------------------------------------------------------------------------- streaming append
@dataclasses.dataclass
class StreamState:
    """A cache after a run of appends: whole B-token blocks quantized, the rest at full precision."""
    cached: int                   # tokens appended per sequence so far
    quantized: Quantized | None   # the whole blocks, [seqs * whole, heads, D] (None when there is none)
    residual: np.ndarray          # the trailing cached - whole tokens, [seqs, r, heads, D] float64


def stream_state(x_hist: np.ndarray, spec: Spec, signs: np.ndarray | None = None) -> StreamState:
    """The cache after every token of x_hist ([seqs, n, heads, D]) has been appended, by any
    number of appends of any sizes (NSNQuant summary, "implementation details": the cache is a
    quantized part plus a full-precision residual; a residual that fills up is quantized and
    joins the quantized part).

    With per-channel scales a block can only be quantized once all its B tokens are there, so
    the quantized part is the floor(n / B) whole blocks, quantized exactly as quantize() does a
    cache of that many tokens, and the residual is the last n mod B tokens, unchanged.
    """
    x_hist = np.asarray(x_hist, dtype=np.float64)
    S, n, Hh, D = x_hist.shape
    assert spec.per_channel and Hh == spec.heads and D == spec.head_dim
    B = spec.block_tokens
    whole = (n // B) * B
    qz = None
    if whole:
        qz = quantize(x_hist[:, :whole].reshape(S * whole, Hh, D), dataclasses.replace(spec, seqs=S, tokens=whole), signs)
    return StreamState(cached=n, quantized=qz, residual=x_hist[:, whole:].copy())


def attention_decode_stream(q: np.ndarray, k_hat: np.ndarray | None, v_hat: np.ndarray | None,
                            k_res: np.ndarray, v_res: np.ndarray, spec: Spec) -> np.ndarray:
    """Decode attention over a streamed cache, in float64: one softmax over the Tq dequantized
    cached tokens (k_hat, v_hat: [seqs * Tq, heads, D], or None when Tq = 0) followed by the r
    residual tokens at full precision (k_res, v_res: [seqs, r, heads, D]); otherwise exactly
    attention_decode (scores q . k / sqrt(D), query head hq reads KV head hq // G)."""
    q = np.asarray(q, dtype=np.float64)
    S = q.shape[0]
    Hh, D = spec.heads, spec.head_dim
    r = k_res.shape[1]
    Tq = 0 if k_hat is None else k_hat.shape[0] // S
    parts_k = [np.asarray(k_res, dtype=np.float64)]
    parts_v = [np.asarray(v_res, dtype=np.float64)]
    if Tq:
        parts_k.insert(0, np.asarray(k_hat, dtype=np.float64).reshape(S, Tq, Hh, D))
        parts_v.insert(0, np.asarray(v_hat, dtype=np.float64).reshape(S, Tq, Hh, D))
    kk = np.concatenate(parts_k, axis=1).reshape(S * (Tq + r), Hh, D)
    vv = np.concatenate(parts_v, axis=1).reshape(S * (Tq + r), Hh, D)
    return attention_decode(q, kk, vv, dataclasses.replace(spec, seqs=S, tokens=Tq + r))


# ----------------------------------------------------------------------------- error report
# ----------------------------------------------------------------------------- RRS INT4 GEMM
RRS_GROUP = 128     # channels per runtime-smoothing group = the GEMM's K block (Figure 4)


@dataclasses.dataclass
class RrsActivations:
    codes: np.ndarray      # int8 [N, K] in [-Q, Q]
    packed: np.ndarray     # uint8 [N, K/2]
    v: np.ndarray          # float64 quotient before rounding [N, K]
    scale: np.ndarray      # float64 per-token scale a_t [N]
    scales16: np.ndarray   # float16 stored a_t


def rrs_smooth_scales(x: np.ndarray, signs: np.ndarray | None, hadamard: int, group: int = RRS_GROUP) -> np.ndarray:
    """Runtime smoothing scales (Rotated Runtime Smooth analysis, "master equation" and
    "term-by-term": s_j = the largest |(X R)_tj| over the N tokens of column j; Figure 4: the
    group of `group` channels takes its largest s_j).  x: [N, K]; returns s [K / group] float64."""
    x = np.asarray(x, dtype=np.float64)
    N, K = x.shape
    y = rotate(x[:, None, :], signs[None, :], hadamard)[:, 0, :] if hadamard else x
    col = np.abs(y).max(axis=0) if N else np.zeros(K)
    return col.reshape(K // group, group).max(axis=1)


def rrs_quantize_act(x: np.ndarray, signs: np.ndarray | None, hadamard: int, s: np.ndarray, bits: int = 4,
                     group: int = RRS_GROUP) -> RrsActivations:
    """X'_quant = Quantize(X R diag(s)^-1) ("master equation"): every column of the rotated
    activations divided by its group's smoothing scale, then symmetric per-token INT-b with
    round-to-nearest (the per-token absmax reading of the activation quantizer), rounding the
    quotient half to even as for the cache modes."""
    x = np.asarray(x, dtype=np.float64)
    N, K = x.shape
    Q = qmax(bits)
    y = rotate(x[:, None, :], signs[None, :], hadamard)[:, 0, :] if hadamard else x
    sc = np.repeat(np.asarray(s, dtype=np.float64), group)
    u = np.where(sc[None, :] > 0.0, y / np.where(sc > 0.0, sc, 1.0)[None, :], 0.0)
    a = np.abs(u).max(axis=1) / Q if K else np.zeros(N)
    safe = np.where(a > 0.0, a, 1.0)
    v = np.where(a[:, None] > 0.0, u / safe[:, None], 0.0)
    # near a tie, the exact quotient: Q (Y_c / s_g(c)) / max_c' |Y_c' / s_g(c')| (1/sqrt(n) cancels)
    sfr = [Fraction(float(e)) for e in np.asarray(s, dtype=np.float64)]
    rows = {}

    def smoothed(t):
        if t not in rows:
            yv = _exact_rotation(x[t], signs, hadamard)
            rows[t] = [yv[j] / sfr[j // group] if sfr[j // group] else Fraction(0) for j in range(K)]
        return rows[t]

    def exact_square(idx):
        t, j = (int(i) for i in idx)
        z = smoothed(t)
        return (1 if z[j] > 0 else -1), Fraction(Q * Q) * z[j] ** 2 / max(e * e for e in z)

    c = _round_codes(v, Q, exact_square)
    return RrsActivations(codes=c, packed=pack_nibbles(c), v=v, scale=a, scales16=a.astype(np.float16))


def rrs_quantize_weights(w: np.ndarray, signs: np.ndarray | None, hadamard: int, bits: int = 4) -> Quantized:
    """W'_quant = Quantize(W_rot): every weight row rotated as the activation rows are (W_rot =
    W R keeps X W^T = X_rot W_rot^T; the page's R^-1 W does not type-check for an M x K weight),
    then symmetric per-output-channel INT-b with round-to-nearest: the per-token NAIVE mode
    with each of the M rows as one token."""
    w = np.asarray(w, dtype=np.float64)
    M, K = w.shape
    spec = Spec(1, M, 1, K, bits, "naive", M, hadamard)
    return quantize(w[:, None, :], spec, None if signs is None else signs[None, :])


def rrs_gemm(x_codes: np.ndarray, a16: np.ndarray, w_codes: np.ndarray, b16: np.ndarray, s: np.ndarray,
             group: int = RRS_GROUP) -> np.ndarray:
    """Y = sum_j (X'_quant)_j (W'_quant)_j^T s_j ("master equation", the channel sum of the
    term-by-term analysis): with X'_quant = a_t c_tj and W'_quant = b_m d_mj and s_j shared by
    a group, Y_tm = a_t b_m sum_g s_g sum_{j in g} c_tj d_mj; each group's integer product is
    exact and the scale is applied to it (Figure 4: scales on the interim results).  float64."""
    c = np.asarray(x_codes, dtype=np.int64)
    d = np.asarray(w_codes, dtype=np.int64)
    N, K = c.shape
    M = d.shape[0]
    acc = np.zeros((N, M))
    for g in range(K // group):
        part = c[:, g * group:(g + 1) * group] @ d[:, g * group:(g + 1) * group].T     # exact integers
        acc += part.astype(np.float64) * float(s[g])
    return acc * np.asarray(a16, dtype=np.float64)[:, None] * np.asarray(b16, dtype=np.float64)[None, :]


def reconstruction_errors(x: np.ndarray, x_hat: np.ndarray, outlier_mask: np.ndarray) -> dict:
    """Four relative-error measures of a reconstruction (for the mode ordering check).

    outlier_mask: bool [heads, D], True on the generator's outlier channels.
    """
    x = np.asarray(x, dtype=np.float64)
    err = x_hat - x
    fro = np.linalg.norm(err) / np.linalg.norm(x)
    tok = np.mean(np.linalg.norm(err, axis=-1) / np.maximum(np.linalg.norm(x, axis=-1), 1e-300))
    ch = np.mean(np.linalg.norm(err, axis=0) / np.maximum(np.linalg.norm(x, axis=0), 1e-300))
    keep = ~outlier_mask[None, :, :]
    keep = np.broadcast_to(keep, x.shape)
    non = np.linalg.norm(err[keep]) / np.linalg.norm(x[keep])
    return {"frobenius": fro, "per_token": tok, "per_channel": ch, "non_outlier": non}
