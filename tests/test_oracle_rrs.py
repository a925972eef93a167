"""Pins of the oracle's RRS activation path into an INT4 GEMM (Rotated Runtime Smooth analysis,
"master equation", "term-by-term", "step-by-step flow", Figure 4).

Each pin checks rrs_smooth_scales / rrs_quantize_act / rrs_quantize_weights / rrs_gemm against
something other than the oracle's own code: a dense rotation matrix built entry by entry, integer
grid inputs on which quantization is exact (so Y must equal X W^T), the invariance of Y under a
reordering of whole channel groups, and scalar loops.
"""
import numpy as np

import oracle

G = oracle.RRS_GROUP


def _dense_rotation(signs, n):
    """R with X_rot = X R: block-diagonal, entry (c, c') = sigma_c H[c' % n, c % n] / sqrt(n) inside
    a block, written out entry by entry."""
    K = signs.shape[0]
    R = np.zeros((K, K))
    for c in range(K):
        for cp in range(K):
            if c // n == cp // n:
                h = -1.0 if bin((c % n) & (cp % n)).count("1") % 2 else 1.0
                R[c, cp] = signs[c] * h / np.sqrt(n)
    return R


def _signs(rng, K):
    return rng.choice(np.array([-1, 1], np.int8), size=K)


def test_smooth_scales_against_a_dense_rotation():
    rng = np.random.default_rng(1)
    N, K = 5, 2 * G
    x = rng.standard_normal((N, K)) * rng.uniform(0.1, 10.0, size=(1, K))
    sg = _signs(rng, K)
    xr = x @ _dense_rotation(sg, G)
    want = np.array([max(abs(xr[t, j]) for t in range(N) for j in range(g * G, (g + 1) * G)) for g in range(K // G)])
    np.testing.assert_allclose(oracle.rrs_smooth_scales(x, sg, G), want, rtol=1e-12)


def _grid_problem(rng, N, M, K, had=True):
    """X, W whose rotations are integer grids: X R = Z diag(2^e) (e per group), W R = V, every row
    of Z and V and every group of Z holding a +-7.  Then s_g = 7 2^e_g, a_t = 1/7, b_m = 1 and the
    codes are Z and V exactly."""
    Z = rng.integers(-7, 8, size=(N, K))
    Z[np.arange(N), rng.integers(0, K, size=N)] = 7 * rng.choice([-1, 1], size=N)
    for g in range(K // G):
        Z[rng.integers(0, N), g * G + rng.integers(0, G)] = -7
    V = rng.integers(-7, 8, size=(M, K))
    V[np.arange(M), rng.integers(0, K, size=M)] = 7
    e = rng.integers(-3, 4, size=K // G)
    Y = Z * np.repeat(2.0 ** e, G)[None, :]
    sg = _signs(rng, K) if had else None
    if had:
        X = oracle.inverse_rotate(Y[:, None, :], sg[None, :], G)[:, 0, :]
        W = oracle.inverse_rotate(V.astype(np.float64)[:, None, :], sg[None, :], G)[:, 0, :]
    else:
        X, W = Y, V.astype(np.float64)
    return X, W, sg, Z, V, e


def test_grid_inputs_give_exact_codes_and_the_exact_product():
    rng = np.random.default_rng(2)
    N, M, K = 9, 6, 3 * G
    X, W, sg, Z, V, e = _grid_problem(rng, N, M, K)
    s = oracle.rrs_smooth_scales(X, sg, G)
    np.testing.assert_allclose(s, 7.0 * 2.0 ** e, rtol=1e-12)
    act = oracle.rrs_quantize_act(X, sg, G, s)
    wq = oracle.rrs_quantize_weights(W, sg, G)
    np.testing.assert_array_equal(act.codes, Z)
    np.testing.assert_array_equal(wq.codes[:, 0, :], V)
    np.testing.assert_allclose(act.scale, 1.0 / 7.0, rtol=1e-12)
    np.testing.assert_allclose(wq.scale[:, 0], 1.0, rtol=1e-12)
    # with the unrounded scales the grouped, scaled integer product is X W^T itself
    y = oracle.rrs_gemm(act.codes, act.scale, wq.codes[:, 0, :], wq.scale[:, 0], s)
    np.testing.assert_allclose(y, X @ W.T, rtol=1e-12, atol=1e-12 * np.abs(X @ W.T).max())


def test_gemm_against_a_scalar_loop():
    rng = np.random.default_rng(3)
    N, M, K = 3, 4, 2 * G
    c = rng.integers(-7, 8, size=(N, K))
    d = rng.integers(-7, 8, size=(M, K))
    a = rng.uniform(0.1, 2.0, size=N)
    b = rng.uniform(0.1, 2.0, size=M)
    s = rng.uniform(0.5, 30.0, size=K // G)
    want = np.zeros((N, M))
    for t in range(N):
        for m in range(M):
            want[t, m] = sum(float(c[t, j]) * float(d[m, j]) * s[j // G] for j in range(K)) * a[t] * b[m]
    np.testing.assert_allclose(oracle.rrs_gemm(c, a, d, b, s), want, rtol=1e-13)


def test_reordering_whole_groups_leaves_y_unchanged():
    # Figure 4's note: Y is a sum over channels, so the order of the groups does not matter
    rng = np.random.default_rng(4)
    N, M, K = 16, 8, 4 * G
    x = rng.standard_normal((N, K))
    x[:, 5] *= 40.0                                   # an outlier channel
    w = rng.standard_normal((M, K)) * 0.05
    sg = _signs(rng, K)
    perm = np.concatenate([np.arange(g * G, (g + 1) * G) for g in (2, 0, 3, 1)])

    def run(xx, ww, ss):
        s = oracle.rrs_smooth_scales(xx, ss, G)
        act = oracle.rrs_quantize_act(xx, ss, G, s)
        wq = oracle.rrs_quantize_weights(ww, ss, G)
        return oracle.rrs_gemm(act.codes, act.scales16, wq.codes[:, 0, :], wq.scales16[:, 0], s), act

    y0, a0 = run(x, w, sg)
    y1, a1 = run(x[:, perm], w[:, perm], sg[perm])
    np.testing.assert_array_equal(a1.codes, a0.codes[:, perm])
    np.testing.assert_allclose(y1, y0, rtol=1e-12, atol=1e-12 * np.abs(y0).max())


def test_smoothing_and_code_ranges():
    rng = np.random.default_rng(5)
    N, K = 32, 2 * G
    x = rng.standard_normal((N, K)) * np.exp(rng.standard_normal((N, 1)))
    x[:, 17] *= 80.0
    sg = _signs(rng, K)
    s = oracle.rrs_smooth_scales(x, sg, G)
    act = oracle.rrs_quantize_act(x, sg, G, s, bits=4)
    xr = oracle.rotate(x[:, None, :], sg[None, :], G)[:, 0, :]
    u = xr / np.repeat(s, G)[None, :]
    # the smoothed activations lie in [-1, 1], each group reaching 1 in some token
    assert np.abs(u).max() <= 1.0 + 1e-15
    np.testing.assert_allclose(np.abs(u).reshape(N, K // G, G).max(axis=(0, 2)), 1.0, rtol=1e-15)
    # every token's codes reach +-Q and stay within it; a_t c is within half a step of u
    assert np.all(np.abs(act.codes).max(axis=1) == 7) and np.abs(act.codes).max() <= 7
    assert np.all(np.abs(act.scale[:, None] * act.codes - u) <= act.scale[:, None] * (0.5 + 1e-6))


def test_without_rotation_the_weight_codes_are_a_row_absmax_rounding():
    rng = np.random.default_rng(6)
    M, K = 5, G
    w = rng.standard_normal((M, K))
    wq = oracle.rrs_quantize_weights(w, None, 0, bits=3)
    for m in range(M):
        b = max(abs(w[m])) / 3.0
        for j in range(K):
            assert wq.codes[m, 0, j] == int(np.rint(np.float32(w[m, j] / b)))
