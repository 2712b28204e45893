"""Pins for the oracle's block decoder and matrix assembly.

Pinned by: the hand-worked block (golden fixture), special cases that reduce to
a column of U or to zero, the power-of-two exponent law, linearity in t, the
exact-in-fp32 bound, and exact rational (Fraction) arithmetic on small cases.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import seedlm_oracle as O


def test_hand_worked_block(golden):
    g = golden("block_seed1.txt")
    seed = int(g["seed"][0])
    t = [int(v) for v in g["t"]]
    e = int(g["e"][0])
    want = np.array([float(v) for v in g["w"]])
    got = O.decode_block(seed, t, e, 8, 3)
    assert np.array_equal(got, want)
    # and the integer form I_i = w_i * 2^(15 - e)
    I = [int(v) for v in g["I"]]
    assert [int(v) for v in got * 2.0 ** (15 - e)] == I


def test_zero_coefficients_give_zero_weights():
    for seed in (1, 2, 777, 65535):
        assert np.all(O.decode_block(seed, [0, 0, 0], -3, 8, 3) == 0)
        assert np.all(O.decode_block(seed, [0, 0, 0, 0], 0, 12, 4) == 0)


def test_unit_coefficient_returns_a_column_of_states():
    # t = e_j, e = 0  ->  w_i = (z_{jC+i} - 2^15) / 2^15
    seed = 4242
    for C, P in ((8, 3), (12, 4)):
        z = O.lfsr_states(seed, C * P)
        for j in range(P):
            t = [0] * P
            t[j] = 1
            w = O.decode_block(seed, t, 0, C, P)
            want = [(z[j * C + i] - 32768) / 32768 for i in range(C)]
            assert list(w) == want


def test_exponent_is_an_exact_power_of_two_scale():
    rng = np.random.default_rng(3)
    for _ in range(20):
        seed = int(rng.integers(1, 65536))
        t = [int(v) for v in rng.integers(-8, 8, 3)]
        w0 = O.decode_block(seed, t, -15, 8, 3)
        for e in range(-14, 1):
            assert np.array_equal(O.decode_block(seed, t, e, 8, 3), w0 * 2.0 ** (e + 15))


def test_linear_in_coefficients():
    rng = np.random.default_rng(4)
    for _ in range(20):
        seed = int(rng.integers(1, 65536))
        a = rng.integers(-4, 4, 4)
        b = rng.integers(-4, 4, 4)
        wa = O.decode_block(seed, list(a), -5, 12, 4)
        wb = O.decode_block(seed, list(b), -5, 12, 4)
        assert np.array_equal(O.decode_block(seed, list(a + b), -5, 12, 4), wa + wb)


def test_weights_are_exact_in_fp32():
    # |I| <= P * 32767 * 8 < 2^24 and the scale 2^(e-15) is a normal fp32 power
    # of two, so every decoded weight is representable in fp32 exactly.
    rng = np.random.default_rng(5)
    for C, P in ((8, 3), (12, 4)):
        for _ in range(50):
            seed = int(rng.integers(1, 65536))
            t = [int(v) for v in rng.integers(-8, 8, P)]
            e = int(rng.integers(-15, 1))
            w = O.decode_block(seed, t, e, C, P)
            assert np.array_equal(w.astype(np.float32).astype(np.float64), w)
    assert 3 * 32767 * 8 < 2 ** 24 and 4 * 32767 * 8 < 2 ** 24


def _fraction_block(seed, t, e, C, P):
    # Independent restatement with exact rationals and the step written inline.
    z = seed
    vals = []
    for _ in range(C * P):
        vals.append(Fraction(z - 32768, 32768))
        fb = (z ^ (z >> 2) ^ (z >> 3) ^ (z >> 5)) & 1
        z = (z >> 1) | (fb << 15)
    scale = Fraction(2) ** e
    return [scale * sum(vals[j * C + i] * t[j] for j in range(P)) for i in range(C)]


def test_decode_rows_matches_exact_rationals_with_ragged_tail():
    # cols = 4*12 + 5 -> the last 3-bit block keeps 5 of its 12 weights.
    rng = np.random.default_rng(11)
    for C, P, cols in ((8, 3, 37), (12, 4, 53)):
        rows = 3
        nb = -(-cols // C)
        seeds = rng.integers(1, 65536, (rows, nb)).astype(np.uint16)
        coeffs = rng.integers(-8, 8, (rows, nb, P)).astype(np.int8)
        exps = rng.integers(-15, 1, (rows, nb)).astype(np.int8)
        W = O.decode_rows(seeds, coeffs, exps, cols, C, P)
        assert W.shape == (rows, cols)
        for r in range(rows):
            full = []
            for b in range(nb):
                full += _fraction_block(int(seeds[r, b]), [int(v) for v in coeffs[r, b]],
                                        int(exps[r, b]), C, P)
            assert [Fraction(v) for v in W[r]] == full[:cols]


def test_decode_rows_rejects_bad_records():
    seeds = np.ones((2, 2), np.uint16)
    coeffs = np.zeros((2, 2, 3), np.int8)
    exps = np.zeros((2, 2), np.int8)
    O.decode_rows(seeds, coeffs, exps, 16, 8, 3)
    with pytest.raises(ValueError):
        O.decode_rows(seeds * 0, coeffs, exps, 16, 8, 3)
    bad = coeffs.copy()
    bad[0, 0, 0] = 8
    with pytest.raises(ValueError):
        O.decode_rows(seeds, bad, exps, 16, 8, 3)
    bad = exps.copy()
    bad[1, 1] = 1
    with pytest.raises(ValueError):
        O.decode_rows(seeds, coeffs, bad, 16, 8, 3)
    bad[1, 1] = -16
    with pytest.raises(ValueError):
        O.decode_rows(seeds, coeffs, bad, 16, 8, 3)
