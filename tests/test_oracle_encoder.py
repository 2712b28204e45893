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


@pytest.mark.parametrize("Q", [3, 4])
def test_quantize_exponent_rule_by_thresholds(Q):
    """Q-bit integers in [-2^(Q-1), 2^(Q-1)-1]; round-half-even keeps t*/2^e in
    range exactly when t*/2^e < 2^(Q-1) - 1/2 and t*/2^e >= -(2^(Q-1) + 1/2), so
    the chosen e is the smallest one in [-15, 0] meeting both (else 0)."""
    rng = np.random.default_rng(Q)
    ts = rng.standard_normal((2000, 3)) * np.exp2(rng.uniform(-16, 4, (2000, 1)))
    t, e = O.quantize(ts, Q)
    half = 1 << (Q - 1)
    for v, tv, ev in zip(ts, t, e):
        want = 0
        for cand in range(-15, 1):
            y = v / 2.0 ** cand
            if y.max() < half - 0.5 and y.min() >= -(half + 0.5):
                want = cand
                break
        assert ev == want
        assert tv.min() >= -half and tv.max() <= half - 1
    # boundary cases, Q = 3: 3.5 rounds to 4 (does not fit at e = 0: clamp to 3);
    # -4.5 rounds to -4 (fits at e = 0)
    if Q == 3:
        t1, e1 = O.quantize(np.array([[3.5, 0.0, 0.0]]), 3)
        assert e1[0] == 0 and t1[0, 0] == 3
        t2, e2 = O.quantize(np.array([[-4.5, 0.0, 0.0]]), 3)
        assert e2[0] == 0 and t2[0, 0] == -4


def test_planted_blocks_reencode_exactly_12bit_seeds():
    """The K = 12 search (4095 seeds) returns planted records exactly."""
    rng = np.random.default_rng(12)
    n, C, P, K = 6, 7, 3, 12
    seeds = rng.integers(1, 1 << K, (1, n))
    coeffs = rng.integers(-8, 8, (1, n, P)).astype(np.int8)
    coeffs[0, :, 0] = 7
    exps = rng.integers(-12, -5, (1, n)).astype(np.int8)
    W = O.decode_rows(seeds, coeffs, exps, n * C, C, P, K)
    s2, c2, e2, rec, err = O.encode_exhaustive(W, C, P, K=K)
    assert np.all(err == 0)
    assert np.array_equal(s2.reshape(-1), seeds.reshape(-1))
    assert np.array_equal(O.decode_rows(s2, c2, e2, n * C, C, P, K), W)
