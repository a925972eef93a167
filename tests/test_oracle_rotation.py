"""Pins of the oracle's rotation (reading R1) against things other than itself."""
import numpy as np
import pytest
import scipy.linalg

import oracle


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_is_sylvester_natural_order(n):
    # scipy builds H_n by the Sylvester recursion [[H, H], [H, -H]] -- an independent routine
    np.testing.assert_array_equal(oracle.hadamard_matrix(n), scipy.linalg.hadamard(n))


@pytest.mark.parametrize("n", [2, 16, 128, 256])
def test_hadamard_rows_orthogonal(n):
    H = oracle.hadamard_matrix(n)
    np.testing.assert_array_equal(H @ H.T, n * np.eye(n))


@pytest.mark.parametrize("n", [2, 4, 8, 16])
def test_rotation_brute_force_small(n):
    # explicit loops over the definition y_i = n^-1/2 sum_j H_ij sigma_j x_j, H from scipy
    rng = np.random.default_rng(n)
    D, heads = 2 * n, 3
    x = rng.standard_normal((5, heads, D))
    signs = rng.choice([-1, 1], size=(heads, D)).astype(np.int8)
    Hs = scipy.linalg.hadamard(n)
    want = np.zeros_like(x)
    for t in range(5):
        for h in range(heads):
            for blk in range(D // n):
                for i in range(n):
                    acc = 0.0
                    for j in range(n):
                        d = blk * n + j
                        acc += Hs[i, j] * signs[h, d] * x[t, h, d]
                    want[t, h, blk * n + i] = acc / np.sqrt(n)
    np.testing.assert_allclose(oracle.rotate(x, signs, n), want, rtol=0, atol=1e-13)


def test_rotation_small_integers_exact():
    # with small-integer x the unnormalized transform is exact: H (H x) = n x
    rng = np.random.default_rng(1)
    n = 16
    x = rng.integers(-9, 10, size=(4, 1, n)).astype(np.float64)
    ones = np.ones((1, n), dtype=np.int8)
    y = oracle.rotate(x, ones, n) * 4.0          # 1/sqrt(16) = 1/4 exactly
    back = oracle.rotate(y, ones, n) * 4.0
    np.testing.assert_array_equal(back, n * x)


@pytest.mark.parametrize("n", [16, 64, 128])
def test_parseval_and_inverse(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((7, 2, 256))
    signs = rng.choice([-1, 1], size=(2, 256)).astype(np.int8)
    y = oracle.rotate(x, signs, n)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(oracle.inverse_rotate(y, signs, n), x, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [16, 128])
def test_spike_spreads_evenly(n):
    # a single spike A e_k maps to entries of magnitude exactly A / sqrt(n) (the spreading
    # effect the rotation methods rely on)
    A = 50.0
    signs = np.random.default_rng(0).choice([-1, 1], size=(1, n)).astype(np.int8)
    for k in (0, 5, n - 1):
        x = np.zeros((1, 1, n))
        x[0, 0, k] = A
        y = oracle.rotate(x, signs, n)
        np.testing.assert_allclose(np.abs(y), A / np.sqrt(n), rtol=1e-15)


def test_block_diagonal_uses_its_sign_segment():
    # D = 4096 with n = 128: block k only mixes channels [128k, 128k+128) with sigma[128k:..]
    rng = np.random.default_rng(7)
    n, D = 128, 4096
    signs = rng.choice([-1, 1], size=(1, D)).astype(np.int8)
    for k in (0, 13, 31):
        x = np.zeros((1, 1, D))
        x[0, 0, k * n:(k + 1) * n] = rng.standard_normal(n)
        y = oracle.rotate(x, signs, n)
        mask = np.ones(D, bool)
        mask[k * n:(k + 1) * n] = False
        assert np.all(y[0, 0, mask] == 0.0)
        seg = x[0, 0, k * n:(k + 1) * n] * signs[0, k * n:(k + 1) * n]
        want = scipy.linalg.hadamard(n) @ seg / np.sqrt(n)
        np.testing.assert_allclose(y[0, 0, k * n:(k + 1) * n], want, rtol=0, atol=1e-13)


def test_rotation_preserves_dot_products():
    # Y = (X R)(R^-1 W^T) = X W^T: q . k is unchanged when both are rotated
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    signs = rng.choice([-1, 1], size=(1, 128)).astype(np.int8)
    lhs = float(np.sum(oracle.rotate(q, signs, 128) * oracle.rotate(k, signs, 128)))
    assert abs(lhs - float(np.sum(q * k))) < 1e-12
