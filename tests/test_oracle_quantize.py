"""Pins of the oracle's norm separation, scales, codes and dequantization (C2-C6)."""
import numpy as np
import pytest

import oracle
from oracle import Spec
from tests import grid


def test_norm_is_l2_not_lminus1():
    # (3, 4) has L2 norm 5; the L_{-1} "norm" of the .norm() pitfall would give 12/7
    x = np.zeros((1, 1, 64))
    x[0, 0, 0], x[0, 0, 1] = 3.0, 4.0
    q = oracle.quantize(x, Spec(1, 1, 1, 64, 4, "nsep"))
    assert q.nu[0, 0] == 5.0
    assert q.norms16[0, 0] == np.float16(5.0)


@pytest.mark.parametrize("mode", ["nsep", "nsep_pchan"])
def test_direction_is_unit(mode):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((128, 2, 64)) * rng.uniform(0.2, 5.0, size=(128, 1, 1))
    sp = Spec(1, 128, 2, 64, 4, mode, 64 if mode == "nsep_pchan" else 0)
    q = oracle.quantize(x, sp)
    scale_full = (np.repeat(q.scale.reshape(2, 1, 2, 64), 64, axis=1).reshape(128, 2, 64)
                  if sp.per_channel else q.scale[..., None])
    u = q.v * scale_full
    np.testing.assert_allclose(np.linalg.norm(u, axis=-1), 1.0, rtol=0, atol=1e-12)


def test_rounding_is_half_to_even():
    # exact ties built on the grid: per-token absmax 7 * 2^p, Q = 7 -> quotient = value / 2^p
    vals = np.array([7.0, 0.5, 1.5, 2.5, -2.5, 3.5, 4.5, 5.5, 6.5, -0.5, -1.5, -6.5,
                     0.25, 2.75, -3.25, 1.0])
    x = np.zeros((1, 1, 64))
    x[0, 0, :vals.size] = vals * 2.0 ** -3
    q = oracle.quantize(x, Spec(1, 1, 1, 64, 4, "naive"))
    # Python's round() is round-half-even (an independent library routine)
    want = [round(float(v)) for v in vals]
    np.testing.assert_array_equal(q.codes[0, 0, :vals.size], want)
    # ... and it differs from half-away-from-zero on these inputs
    away = np.sign(vals) * np.floor(np.abs(vals) + 0.5)
    assert np.any(away != np.array(want))


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("mode", oracle.MODES)
def test_codes_in_range_and_no_0x8_nibble(bits, mode):
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((256, 2, 64)) * 3
    x[:, :, 5] *= 40
    sp = Spec(2, 128, 2, 64, bits, mode, 64 if "pchan" in mode else 0)
    q = oracle.quantize(x, sp)
    Q = oracle.qmax(bits)
    assert q.codes.min() >= -Q and q.codes.max() <= Q
    assert not np.any((q.packed & 0xF) == 8) and not np.any((q.packed >> 4) == 8)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("mode", oracle.MODES)
def test_every_scale_group_reaches_q(bits, mode):
    # the group's absmax element lands exactly on +-Q: catches a wrong reduction axis
    rng = np.random.default_rng(10 + bits)
    x = rng.standard_normal((2 * 128, 3, 64)) * rng.uniform(0.3, 3.0, size=(256, 1, 1))
    B = 32
    sp = Spec(2, 128, 3, 64, bits, mode, B if "pchan" in mode else 0)
    q = oracle.quantize(x, sp)
    Q = oracle.qmax(bits)
    a = np.abs(q.codes.astype(int))
    if sp.per_channel:
        m = a.reshape(2, 128 // B, B, 3, 64).max(axis=2)
    else:
        m = a.max(axis=-1)
    assert np.all(m == Q)


def test_per_channel_scale_brute_force():
    # explicit loops: scale[s*nb + b, h, d] = max over tokens of block b of |u| / Q
    rng = np.random.default_rng(5)
    S, T, H, D, B = 2, 8, 2, 4 * 2, 4
    x = rng.standard_normal((S * T, H, D))
    sp = Spec(S, T, H, D, 4, "nsep_pchan", B)
    q = oracle.quantize(x, sp)
    for s in range(S):
        for b in range(T // B):
            for h in range(H):
                for d in range(D):
                    best = 0.0
                    for t in range(b * B, (b + 1) * B):
                        row = x[s * T + t, h]
                        nrm = sum(float(e) * float(e) for e in row) ** 0.5
                        best = max(best, abs(row[d]) / nrm)
                    assert abs(q.scale[s * (T // B) + b, h, d] - best / 7) < 1e-15


def test_nsep_gives_naive_codes():
    # (y/nu) / (max|y|/nu / Q) = y Q / max|y|: norm separation alone leaves codes unchanged
    rng = np.random.default_rng(2)
    x = rng.standard_normal((512, 4, 128)) * rng.uniform(0.2, 5.0, size=(512, 1, 1))
    for bits in (2, 3, 4):
        a = oracle.quantize(x, Spec(1, 512, 4, 128, bits, "naive"))
        b = oracle.quantize(x, Spec(1, 512, 4, 128, bits, "nsep"))
        diff = a.codes != b.codes
        # only possible where the fp64 quotients straddle a tie by rounding noise
        frac = np.abs(np.abs(a.v[diff]) % 1.0 - 0.5)
        assert np.all(frac < 1e-9)
        assert diff.mean() < 1e-5


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("mode", oracle.MODES)
@pytest.mark.parametrize("had", [0, 16, 64])
def test_grid_inputs_round_trip_exactly(bits, mode, had):
    sp, x, signs, want_codes = grid.make(bits, mode, had, head_dim=64, seed=bits * 7 + had)
    q = oracle.quantize(x, sp, signs)
    np.testing.assert_array_equal(q.codes, want_codes)
    xh = oracle.dequantize(q.packed, q.norms16, q.scales16, sp, signs)
    np.testing.assert_array_equal(xh, x)


@pytest.mark.parametrize("mode", oracle.MODES)
def test_dequant_error_within_half_step(mode):
    # in the rotated domain |y^ - y| <= scale * nu / 2, up to the fp16 storage of scale/norm
    rng = np.random.default_rng(4)
    x = rng.standard_normal((256, 2, 128)) * rng.uniform(0.3, 3.0, size=(256, 1, 1))
    x[:, :, 9] *= 30
    signs = rng.choice([-1, 1], size=(2, 128)).astype(np.int8)
    sp = Spec(2, 128, 2, 128, 4, mode, 64 if "pchan" in mode else 0, 128)
    q = oracle.quantize(x, sp, signs)
    y = oracle.rotate(x, signs, 128)
    sp0 = Spec(2, 128, 2, 128, 4, mode, sp.block_tokens, 0)
    yh = oracle.dequantize(q.packed, q.norms16, q.scales16, sp0)
    step = oracle.expand_scales(q.scale, sp) * (q.nu[..., None] if sp.nsep else 1.0)
    stored = oracle.expand_scales(q.scales16, sp) * (q.norms16.astype(np.float64)[..., None] if sp.nsep else 1.0)
    bound = 0.5 * step + np.abs(q.codes) * np.abs(stored - step) + 1e-12
    assert np.all(np.abs(yh - y) <= bound)


@pytest.mark.parametrize("had", [0, 16])
@pytest.mark.parametrize("mode", oracle.MODES)
def test_all_ties_round_half_even(mode, had):
    # every quotient an exact half-integer: codes must be Python's half-even round() of it
    x, signs, want = grid.all_ties(had)
    sp = Spec(1, 128, 2, 64, 4, mode, 64 if "pchan" in mode else 0, had)
    np.testing.assert_array_equal(oracle.quantize(x, sp, signs).codes, want)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("mode", oracle.MODES)
def test_near_ties_round_the_exact_quotient(bits, mode):
    # quotients within ~2^-26 of a tie (2.5 or 0.5), above and below it: the code is the half-even
    # rounding of the exact quotient (rational arithmetic in tests/grid.py), so the tie's two
    # neighbours are told apart; a decision on the fp32 quotient would round both to the tie
    per_channel = "pchan" in mode
    x, signs, want = grid.near_ties(bits, per_channel)
    sp = Spec(1, 64, 1, 64, bits, mode, 64 if per_channel else 0, 16)
    q = oracle.quantize(x, sp, signs)
    np.testing.assert_array_equal(q.codes, want)
    tie = 0.5 if bits == 2 else 2.5
    up = 1 if bits == 2 else 3
    # channel 1 of token 0 lies just above the tie, channel 3 just below; token 2 is the negation
    # of token 0
    assert want[0, 0, 1] == up and want[0, 0, 3] == up - 1
    assert 0 < q.v[0, 0, 1] - tie < 2.0 ** -24 and 0 < tie - q.v[0, 0, 3] < 2.0 ** -24
    assert want[2, 0, 1] == -up and q.codes[2, 0, 1] == -up
    # an fp32 decision would have returned the tie's even neighbour for both channels
    assert np.rint(np.float32(q.v[0, 0, 1])) == up - 1
