"""Pins for the oracle's matvec: exact rational brute force on small cases and
the float64 error bound (every product and sum of dyadic values)."""
from fractions import Fraction

import numpy as np

from oracle import seedlm_oracle as O


def _exact_y(seeds, coeffs, exps, x, cols, C, P):
    # Brute force: per row, per column, rebuild the weight from the LFSR with
    # exact rationals, multiply by the exact x value and sum.
    rows, nb = seeds.shape
    out = []
    for beta in range(x.shape[0]):
        yrow = []
        for r in range(rows):
            acc = Fraction(0)
            for c in range(cols):
                b, i = divmod(c, C)
                z = int(seeds[r, b])
                states = []
                for _ in range(C * P):
                    states.append(z)
                    fb = (z ^ (z >> 2) ^ (z >> 3) ^ (z >> 5)) & 1
                    z = (z >> 1) | (fb << 15)
                w = sum(Fraction(states[j * C + i] - 32768, 32768) * int(coeffs[r, b, j])
                        for j in range(P)) * Fraction(2) ** int(exps[r, b])
                acc += w * Fraction(float(x[beta, c]))
            yrow.append(acc)
        out.append(yrow)
    return out


def test_gemv_matches_exact_rationals_within_fp64_rounding():
    rng = np.random.default_rng(21)
    for C, P, rows, cols, batch, dt in ((8, 3, 5, 24, 2, np.float16), (12, 4, 4, 30, 1, np.float32)):
        nb = -(-cols // C)
        seeds = rng.integers(1, 65536, (rows, nb)).astype(np.uint16)
        coeffs = rng.integers(-8, 8, (rows, nb, P)).astype(np.int8)
        exps = rng.integers(-12, -5, (rows, nb)).astype(np.int8)
        x = rng.standard_normal((batch, cols)).astype(dt)
        y = O.reference_gemv(seeds, coeffs, exps, x, cols, C, P)
        exact = _exact_y(seeds, coeffs, exps, x, cols, C, P)
        for beta in range(batch):
            scale = max(abs(float(v)) for v in exact[beta])
            for r in range(rows):
                assert abs(y[beta, r] - float(exact[beta][r])) <= 1e-13 * scale


def test_gemv_row_subset_equals_full():
    rng = np.random.default_rng(22)
    rows, cols = 9, 40
    seeds = rng.integers(1, 65536, (rows, 5)).astype(np.uint16)
    coeffs = rng.integers(-8, 8, (rows, 5, 3)).astype(np.int8)
    exps = rng.integers(-12, -5, (rows, 5)).astype(np.int8)
    x = rng.standard_normal((1, cols)).astype(np.float16)
    full = O.reference_gemv(seeds, coeffs, exps, x, cols, 8, 3)
    part = O.reference_gemv(seeds, coeffs, exps, x, cols, 8, 3, rows=[0, 4, 8])
    assert np.array_equal(part, full[:, [0, 4, 8]])


def test_normwise_error_metric():
    assert O.normwise_error([1.0, 2.0], [1.0, 2.0]) == 0.0
    assert O.normwise_error([1.0, 2.5], [1.0, 2.0]) == 0.25
    assert O.normwise_error([0.0], [0.0]) == 0.0
