"""Pins of the oracle's decode attention (softmax over the cache, then the value average)."""
import math

import numpy as np

import oracle
from oracle import Spec


def _spec(T=8, H=2, D=4):
    return Spec(1, T, H, D, 4, "nsep_pchan", 4, 0)


def test_equal_scores_give_the_mean_value():
    # q = 0: every score is 0, softmax is uniform, the output is the plain mean over tokens
    rng = np.random.default_rng(0)
    sp = _spec()
    k = rng.standard_normal((8, 2, 4))
    v = rng.standard_normal((8, 2, 4))
    out = oracle.attention_decode(np.zeros((1, 4, 4)), k, v, sp)
    for hq in range(4):
        np.testing.assert_allclose(out[0, hq], v[:, hq // 2].mean(axis=0), rtol=0, atol=1e-15)


def test_one_dominant_key_selects_its_value():
    sp = _spec()
    k = np.zeros((8, 2, 4))
    k[5, 0, 1] = 1.0                       # only token 5 of head 0 answers q along channel 1
    v = np.arange(8 * 2 * 4, dtype=np.float64).reshape(8, 2, 4)
    q = np.zeros((1, 4, 4))
    q[0, 0, 1] = 2000.0                    # score 1000 after 1/sqrt(4): p ~ 1 on token 5
    out = oracle.attention_decode(q, k, v, sp)
    np.testing.assert_allclose(out[0, 0], v[5, 0], rtol=0, atol=1e-12)


def test_brute_force_loops():
    rng = np.random.default_rng(3)
    S, T, H, D, G = 2, 6, 2, 4, 2
    sp = Spec(S, T, H, D, 4, "nsep", 0, 0)
    k = rng.standard_normal((S * T, H, D))
    v = rng.standard_normal((S * T, H, D))
    q = rng.standard_normal((S, H * G, D))
    out = oracle.attention_decode(q, k, v, sp)
    for s in range(S):
        for hq in range(H * G):
            h = hq // G
            z = [sum(q[s, hq, d] * k[s * T + t, h, d] for d in range(D)) / math.sqrt(D) for t in range(T)]
            e = [math.exp(x - max(z)) for x in z]
            w = [x / sum(e) for x in e]
            for d in range(D):
                want = sum(w[t] * v[s * T + t, h, d] for t in range(T))
                assert abs(out[s, hq, d] - want) < 1e-13


def test_shift_invariance_and_convexity():
    # adding a constant to every score changes nothing; the output lies in the values' hull
    rng = np.random.default_rng(4)
    sp = _spec(T=16)
    k = rng.standard_normal((16, 2, 4))
    v = rng.standard_normal((16, 2, 4))
    q = rng.standard_normal((1, 4, 4))
    out = oracle.attention_decode(q, k, v, sp)
    k2 = k.copy()
    k2[:, :, 0] += 3.0                      # q . k shifts by 3 q[0] for every token of a head
    q2 = q.copy()
    out2 = oracle.attention_decode(q2, k2, v, sp)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-12)
    for hq in range(4):
        vv = v[:, hq // 2]
        assert np.all(out[0, hq] <= vv.max(axis=0) + 1e-12) and np.all(out[0, hq] >= vv.min(axis=0) - 1e-12)
