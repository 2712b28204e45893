"""Encoder self-check: exhaustive 2^16-1 seed search on a 64x64 N(0,1) matrix.

Checks (a) the decoder reproduces the encoder's stored reconstruction bit for
bit, (b) the chosen seed is optimal, recomputed independently for a few blocks
with least squares and an explicit per-seed loop, and (c) planted blocks
re-encode with zero error.
"""
import numpy as np
import pytest

from oracle import seedlm_oracle as O
from workloads import gen_gaussian_matrix


@pytest.fixture(scope="module")
def encoded():
    W = gen_gaussian_matrix(0, 99, 64, 64)
    return W, O.encode_exhaustive(W, 8, 3)


@pytest.mark.slow
def test_decode_of_stored_records_equals_stored_reconstruction(encoded):
    W, (s, c, e, rec, err) = encoded
    assert np.array_equal(O.decode_rows(s, c, e, 64, 8, 3), rec)
    # and the per-block error is the squared distance to W
    blocks = (W - rec).reshape(64, 8, 8)
    assert np.allclose(np.sum(blocks ** 2, axis=-1), err, rtol=1e-12, atol=1e-15)
    # exponents stay in the format's range; coefficients use the 4-bit range
    assert e.min() >= -15 and e.max() <= 0
    assert c.min() >= -8 and c.max() <= 7


def _independent_best(w, C=8, P=3):
    # Per seed: basis from the state list, least squares, shared-exponent
    # quantisation by trying exponents from -15 up, squared error.
    best = (np.inf, None)
    for seed in range(1, 65536):
        z = O.lfsr_states(seed, C * P)
        U = np.array([[(z[j * C + i] - 32768) / 32768 for j in range(P)] for i in range(C)])
        ts = np.linalg.lstsq(U, w, rcond=None)[0]
        e_use = 0
        for e in range(-15, 1):
            q = np.round(ts / 2.0 ** e)
            if np.all(q >= -8) and np.all(q <= 7):
                e_use = e
                break
        t = np.clip(np.round(ts / 2.0 ** e_use), -8, 7)
        r = w - 2.0 ** e_use * (U @ t)
        er = float(r @ r)
        if er < best[0]:
            best = (er, seed)
    return best


@pytest.mark.slow
def test_chosen_seed_is_optimal_for_sampled_blocks(encoded):
    W, (s, c, e, rec, err) = encoded
    for (r, b) in ((0, 0), (37, 5)):
        w = W[r, 8 * b:8 * b + 8]
        best_err, best_seed = _independent_best(w)
        assert err[r, b] <= best_err * (1 + 1e-9) + 1e-15
        assert abs(err[r, b] - best_err) <= 1e-9 * max(best_err, 1e-30)


@pytest.mark.slow
def test_planted_blocks_reencode_exactly():
    rng = np.random.default_rng(2024)
    nblk = 4
    seeds = rng.integers(1, 65536, (1, nblk)).astype(np.uint16)
    coeffs = rng.integers(-8, 8, (1, nblk, 3)).astype(np.int8)
    coeffs[0, :, 0] = 7  # keep max|t| large so the exponent is unique
    exps = rng.integers(-12, -5, (1, nblk)).astype(np.int8)
    W = O.decode_rows(seeds, coeffs, exps, 8 * nblk, 8, 3)
    s2, c2, e2, rec, err = O.encode_exhaustive(W, 8, 3)
    assert np.all(err == 0)
    assert np.array_equal(rec, W)
    assert np.array_equal(O.decode_rows(s2, c2, e2, 8 * nblk, 8, 3), W)
    assert np.array_equal(s2, seeds)
