"""Pins of the oracle's streaming append and of attention over a streamed cache.

The state after a run of appends is fixed by the NSNQuant summary ("implementation details":
a quantized part plus a full-precision residual, flushed into the quantized part when full)
together with per-channel scales needing whole B-token blocks.  The pins check it against
properties a wrong state would break: whole blocks quantize independently of each other,
finished blocks never change, the residual is the exact tail; and attention over a streamed
grid cache (where dequantization is exact) equals a brute-force softmax over the raw tokens
however they are split between the two parts.
"""
import math

import numpy as np

import oracle
from tests import grid


def _outlier_tokens(rng, S, n, H, D):
    x = rng.standard_normal((S, n, H, D))
    x[..., 3] *= 40.0
    return x * rng.uniform(0.3, 3.0, size=(S, n, 1, 1))


def test_whole_blocks_quantize_one_by_one():
    # per-channel scales see only their own block: quantizing three blocks at once equals
    # quantizing each block alone (a scale taken over the whole prefix would fail this)
    rng = np.random.default_rng(1)
    S, B, H, D = 2, 16, 3, 32
    x = _outlier_tokens(rng, S, 3 * B, H, D)
    signs = rng.choice(np.array([-1, 1], np.int8), size=(H, D))
    spec = oracle.Spec(S, 3 * B, H, D, 4, "nsep_pchan", B, 16)
    whole = oracle.quantize(x.reshape(S * 3 * B, H, D), spec, signs)
    c = whole.codes.reshape(S, 3, B, H, D)
    n16 = whole.norms16.reshape(S, 3, B, H)
    s16 = whole.scales16.reshape(S, 3, H, D)
    for b in range(3):
        one = oracle.quantize(x[:, b * B:(b + 1) * B].reshape(S * B, H, D), oracle.Spec(S, B, H, D, 4, "nsep_pchan", B, 16), signs)
        np.testing.assert_array_equal(one.codes.reshape(S, B, H, D), c[:, b])
        np.testing.assert_array_equal(one.norms16.reshape(S, B, H), n16[:, b])
        np.testing.assert_array_equal(one.scales16.reshape(S, H, D), s16[:, b])


def test_stream_state_tail_and_finished_blocks():
    rng = np.random.default_rng(2)
    S, B, H, D = 2, 16, 2, 32
    x = _outlier_tokens(rng, S, 3 * B + 5, H, D)
    spec = oracle.Spec(S, 0, H, D, 4, "pchan", B, 0)
    prev = None
    for n in (0, 1, B - 1, B, B + 1, 2 * B, 3 * B + 5):
        st = oracle.stream_state(x[:, :n], spec)
        whole = (n // B) * B
        assert st.cached == n
        assert (st.quantized is None) == (whole == 0)
        np.testing.assert_array_equal(st.residual, x[:, whole:n])       # the exact tail
        assert st.residual.shape[1] < B
        if st.quantized is not None:
            codes = st.quantized.codes.reshape(S, whole, H, D)
            if prev is not None:
                # blocks finished by an earlier append are never rewritten
                np.testing.assert_array_equal(codes[:, :prev.shape[1]], prev)
            prev = codes


def _brute_attention(q, k, v):
    """softmax(q . k_t / sqrt(D)) v with Python loops; q [S, Hq, D], k, v [S, n, H, D]."""
    S, Hq, D = q.shape
    n, H = k.shape[1], k.shape[2]
    G = Hq // H
    out = np.zeros((S, Hq, D))
    for s in range(S):
        for hq in range(Hq):
            h = hq // G
            sc = [sum(q[s, hq, d] * k[s, t, h, d] for d in range(D)) / math.sqrt(D) for t in range(n)]
            mx = max(sc)
            w = [math.exp(a - mx) for a in sc]
            tot = sum(w)
            for d in range(D):
                out[s, hq, d] = sum(w[t] * v[s, t, h, d] for t in range(n)) / tot
    return out


def test_stream_attention_on_the_grid_matches_brute_force():
    # grid inputs dequantize exactly, so attention over (dequantized whole blocks + residual)
    # must equal plain attention over the raw tokens wherever the split falls
    S, H, D, T = 2, 2, 16, 48
    spec_k, xk, sk, _ = grid.make(4, "nsep_pchan", 16, head_dim=D, seqs=S, tokens=T, heads=H, seed=3)
    _, xv, sv, _ = grid.make(4, "nsep_pchan", 16, head_dim=D, seqs=S, tokens=T, heads=H, seed=4)
    B = spec_k.block_tokens
    k_hist = xk.reshape(S, T, H, D)
    v_hist = xv.reshape(S, T, H, D)
    q = np.random.default_rng(5).standard_normal((S, 2 * H, D))
    for n in (5, B, B + 7, 2 * B - 1, T):
        sk_st = oracle.stream_state(k_hist[:, :n], spec_k, sk)
        sv_st = oracle.stream_state(v_hist[:, :n], spec_k, sv)
        whole = (n // B) * B
        k_hat = v_hat = None
        if whole:
            sp = oracle.Spec(S, whole, H, D, 4, "nsep_pchan", B, 16)
            k_hat = oracle.dequantize(sk_st.quantized.packed, sk_st.quantized.norms16, sk_st.quantized.scales16, sp, sk)
            v_hat = oracle.dequantize(sv_st.quantized.packed, sv_st.quantized.norms16, sv_st.quantized.scales16, sp, sv)
            np.testing.assert_array_equal(k_hat.reshape(S, whole, H, D), k_hist[:, :whole])   # the grid property
        got = oracle.attention_decode_stream(q, k_hat, v_hat, sk_st.residual, sv_st.residual, spec_k)
        want = _brute_attention(q, k_hist[:, :n], v_hist[:, :n])
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
