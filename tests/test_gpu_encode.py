"""GPU seed search (seedlm_encode, through the C ABI) against the CPU oracle.

The oracle's encode_exhaustive scores every seed in float64; the kernel scores
in fp32 (a sum of exact bf16 products accumulated in fp32, then a handful of
fp32 operations per score).  The chosen score is the one thing the search fixes
uniquely, so the bars are on scores, per block with w its weights and
wn = ||w||^2:
  * the kernel's reported score equals the float64 score of its own record
    (recomputed by the oracle's decoder) within 1e-5 * wn: fp32 rounding of a
    few dozen operations on terms of size <= wn stays near 1e-6 * wn;
  * that float64 score is within 1e-5 * wn of the oracle's minimum (a seed the
    kernel prefers by less than its rounding error is as good a choice);
  * records are valid (seed in [1, 2^K - 1], t in [-2^(Q-1), 2^(Q-1) - 1],
    e in [-15, 0]), and
    where the seed agrees with the oracle's, t and e agree too.
Seeds themselves are compared as a rate (they differ only at near-ties).
Small matrices run the oracle on every block; large ones on sampled blocks.
"""
import numpy as np
import pytest

from oracle import seedlm_oracle as O
from workloads import bf16_to_float64, gen_bf16_weights, to_bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCORE_TOL = 1e-5


def _S():
    import prng_seeded_decode_amd as S

    return S


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


_ENCODERS = {}


def _encoder(C, P, K=16, Q=4):
    key = (C, P, K, Q)
    if key not in _ENCODERS:
        _ENCODERS.clear()  # one seed table resident at a time
        _ENCODERS[key] = _S().SeedLMEncoder(C, P, K, Q)
    return _ENCODERS[key]


def _run(bits, C, P, K=16, Q=4):
    """Encode bf16 bit patterns on the GPU; returns host numpy records + scores."""
    dev = _dev()
    W = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    s, c, e, err = _S().seedlm_encode(_encoder(C, P, K, Q), W)
    torch.cuda.synchronize()
    s = s.cpu().numpy().view(np.uint16 if K <= 16 else np.uint32)
    return s, c.cpu().numpy(), e.cpu().numpy(), err.cpu().numpy().astype(np.float64)


def _blocks(W64, C):
    return W64.reshape(-1, C)


def _check_blocks(Wb, s_g, c_g, e_g, err_g, C, P, min_seed_match=0.9, K=16, Q=4):
    """Wb: (k, C) float64 blocks; GPU records for exactly those blocks."""
    k = Wb.shape[0]
    s_g = s_g.reshape(k, 1)
    c_g = c_g.reshape(k, 1, P)
    e_g = e_g.reshape(k, 1)
    err_g = err_g.reshape(k)
    h = 1 << (Q - 1)
    assert s_g.min() >= 1 and int(s_g.max()) <= (1 << K) - 1
    assert c_g.min() >= -h and c_g.max() <= h - 1
    assert e_g.min() >= -15 and e_g.max() <= 0
    wn = np.sum(Wb ** 2, axis=1)
    dec = O.decode_rows(s_g, c_g, e_g, C, C, P, K=K)
    err64 = np.sum((Wb - dec) ** 2, axis=1)
    assert np.all(np.abs(err_g - err64) <= SCORE_TOL * wn + 1e-30), \
        np.max(np.abs(err_g - err64) / np.maximum(wn, 1e-30))
    s_o, c_o, e_o, rec_o, err_o = O.encode_exhaustive(Wb, C, P, K=K, Q=Q)
    err_o = err_o.reshape(k)
    assert np.all(err64 <= err_o + SCORE_TOL * wn + 1e-30), \
        np.max((err64 - err_o) / np.maximum(wn, 1e-30))
    same = s_g.reshape(k) == s_o.reshape(k)
    _say(f"  {k} blocks: seed agreement {same.mean():.4f}, "
         f"max |score - oracle min| / wn {np.max(np.abs(err64 - err_o) / np.maximum(wn, 1e-30)):.2e}")
    assert same.mean() >= min_seed_match
    assert np.array_equal(c_g.reshape(k, P)[same], c_o.reshape(k, P)[same])
    assert np.array_equal(e_g.reshape(k)[same], e_o.reshape(k)[same])


@pytest.mark.parametrize("C,P,rows,cols", [(8, 3, 12, 64), (12, 4, 6, 96)])
def test_encode_small_matches_oracle_on_every_block(C, P, rows, cols):
    _say(f"encode small C={C} {rows}x{cols}")
    bits = gen_bf16_weights(5, C, rows, cols)
    s, c, e, err = _run(bits, C, P)
    _check_blocks(_blocks(bf16_to_float64(bits), C), s, c, e, err, C, P)


@pytest.mark.parametrize("C,P,rows,cols,scale", [(8, 3, 512, 1024, 0.02), (12, 4, 256, 768, 0.02)])
def test_encode_many_workgroups_sampled(C, P, rows, cols, scale):
    """Several hundred workgroups and a ragged last one; every score recomputed
    in float64, sampled blocks against the oracle's exhaustive search."""
    _say(f"encode sampled C={C} {rows}x{cols}")
    bits = gen_bf16_weights(6, C, rows, cols, scale)
    bits = bits[: rows - 3]  # ragged block count
    s, c, e, err = _run(bits, C, P)
    Wb = _blocks(bf16_to_float64(bits), C)
    k = Wb.shape[0]
    wn = np.sum(Wb ** 2, axis=1)
    dec = O.decode_rows(s.reshape(k, 1), c.reshape(k, 1, P), e.reshape(k, 1), C, C, P)
    err64 = np.sum((Wb - dec) ** 2, axis=1)
    assert np.all(np.abs(err.reshape(k) - err64) <= SCORE_TOL * wn)
    # sanity: typical relative error of the best seed (about 0.016 for 4 bits and
    # 0.056 for 3 bits per weight on Gaussian blocks)
    assert np.median(err64 / wn) < (0.03 if C == 8 else 0.08)
    rng = np.random.default_rng(11)
    idx = np.concatenate([[0, k - 1], rng.choice(k, 22, replace=False)])
    _check_blocks(Wb[idx], s.reshape(k)[idx], c.reshape(k, P)[idx], e.reshape(k)[idx],
                  err.reshape(k)[idx], C, P, min_seed_match=0.85)


@pytest.mark.parametrize("C,P", [(8, 3), (12, 4)])
def test_encode_recovers_planted_records(C, P):
    """Blocks made from records, then rounded to bf16.  The planted record stays
    within bf16 rounding of its block, far ahead of a typical seed, so the
    search finds it or a record about as close: after rounding, a few other
    seeds (e.g. one whose column nearly equals the negated planted column) fit
    the block to within the same few parts per million of ||w||^2, and which of
    them wins is decided by rounding (the oracle's float64 and the kernel's fp32
    can differ).  So the bar is the usual score bar, plus the planted seed for
    most blocks."""
    _say(f"encode planted C={C}")
    rng = np.random.default_rng(2025 + C)
    n = 48
    seeds = rng.integers(1, 65536, (1, n)).astype(np.uint16)
    coeffs = rng.integers(-8, 8, (1, n, P)).astype(np.int8)
    coeffs[0, :, 0] = 7  # max |t| large: one exponent fits exactly
    exps = rng.integers(-12, -5, (1, n)).astype(np.int8)
    bits = to_bf16_bits(O.decode_rows(seeds, coeffs, exps, n * C, C, P)).reshape(1, n * C)
    s, c, e, err = _run(bits, C, P)
    _check_blocks(_blocks(bf16_to_float64(bits), C), s, c, e, err, C, P, min_seed_match=0.9)
    planted = s.reshape(-1) == seeds.reshape(-1)
    _say(f"  planted seed recovered for {planted.sum()} of {n} blocks")
    assert planted.mean() >= 0.9
    assert np.array_equal(c.reshape(-1, P)[planted], coeffs.reshape(-1, P)[planted])
    assert np.array_equal(e.reshape(-1)[planted], exps.reshape(-1)[planted])


@pytest.mark.parametrize("C,P", [(8, 3), (12, 4)])
def test_encode_zero_blocks(C, P):
    """A zero block scores 0 with t = 0 for every seed: seed 1 (smallest), e = -15
    (the smallest exponent, at which all-zero coefficients fit)."""
    _say(f"encode zeros C={C}")
    bits = gen_bf16_weights(7, C, 4, 4 * C)
    bits[1] = 0
    bits[3, C:2 * C] = 0
    s, c, e, err = _run(bits, C, P)
    zero = np.zeros((4, 4), bool)
    zero[1] = True
    zero[3, 1] = True
    assert np.all(s[zero] == 1) and np.all(c[zero] == 0) and np.all(e[zero] == -15)
    assert np.all(err[zero] == 0)
    assert np.all(s[~zero] >= 1)


def test_encode_is_deterministic_and_rejects_bad_arguments():
    dev = _dev()
    S = _S()
    bits = gen_bf16_weights(8, 8, 16, 64)
    a = _run(bits, 8, 3)
    b = _run(bits, 8, 3)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    enc = _encoder(8, 3)
    W = torch.zeros((4, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        S.seedlm_encode(enc, torch.zeros((4, 64), dtype=torch.float16, device=dev))
    import ctypes

    L = S.lib()
    out = torch.empty(64, dtype=torch.int32, device=dev)
    p = ctypes.c_void_p(out.data_ptr())
    # misaligned W (C = 8 with cols a multiple of 8 needs 16-byte alignment)
    assert L.seedlm_encode(enc.handle, ctypes.c_void_p(W.data_ptr() + 2), 2, 16, p, p, p, p,
                           None) == S.E_INVALID
    assert L.seedlm_encode(enc.handle, ctypes.c_void_p(W.data_ptr()), 0, 64, p, p, p, p,
                           None) == S.E_INVALID
    assert L.seedlm_encode(enc.handle, ctypes.c_void_p(W.data_ptr()), 4, 0, p, p, p, p,
                           None) == S.E_INVALID
    assert L.seedlm_encode(enc.handle, None, 4, 64, p, p, p, p, None) == S.E_INVALID


# The other formats the encoder is built for (records only: the design-space
# study).  Each is checked on every block of a small Gaussian matrix.
DESIGN_FORMATS = [(6, 1), (7, 2), (9, 4), (10, 5), (11, 6), (12, 7), (8, 1), (9, 1), (10, 2),
                  (11, 3), (8, 2), (8, 4)]


@pytest.mark.parametrize("C,P", DESIGN_FORMATS)
def test_encode_design_space_formats_match_oracle(C, P):
    _say(f"encode format C={C} P={P}")
    bits = gen_bf16_weights(9, 10 * C + P, 2, 12 * C)  # 24 blocks
    s, c, e, err = _run(bits, C, P)
    _check_blocks(_blocks(bf16_to_float64(bits), C), s, c, e, err, C, P, min_seed_match=0.8)


# Other seed widths (the K-bit LFSRs x^12+x^6+x^4+x+1 and x^20+x^3+1) and 3-bit
# coefficients.  K = 20 walks 2^20 - 1 seeds: the oracle's exhaustive search
# takes about half a minute per format there.
SEED_WIDTH_FORMATS = [(7, 3, 12, 4), (8, 2, 12, 4), (9, 3, 20, 4), (12, 3, 20, 4),
                      (8, 4, 16, 3), (10, 3, 16, 3)]


@pytest.mark.parametrize("C,P,K,Q", SEED_WIDTH_FORMATS)
def test_encode_seed_and_coefficient_widths_match_oracle(C, P, K, Q):
    _say(f"encode format C={C} P={P} K={K} Q={Q}")
    bits = gen_bf16_weights(9, 100 * K + 10 * C + P + Q, 2, 12 * C)  # 24 blocks
    s, c, e, err = _run(bits, C, P, K, Q)
    _check_blocks(_blocks(bf16_to_float64(bits), C), s, c, e, err, C, P, min_seed_match=0.8,
                  K=K, Q=Q)


def test_encode_seed_width_planted_records():
    """Blocks made from K = 12 and K = 20 records (seeds past 2^16 for the
    latter, so the wider seed output is exercised), rounded to bf16."""
    for C, P, K in [(7, 3, 12), (9, 3, 20)]:
        _say(f"encode planted C={C} P={P} K={K}")
        rng = np.random.default_rng(77 + K)
        n = 16
        seeds = rng.integers(1, 1 << K, (1, n)).astype(np.uint32)
        if K == 20:
            seeds[0, :8] |= 1 << 16
        coeffs = rng.integers(-8, 8, (1, n, P)).astype(np.int8)
        coeffs[0, :, 0] = 7
        exps = rng.integers(-12, -5, (1, n)).astype(np.int8)
        W = O.decode_rows(seeds, coeffs, exps, n * C, C, P, K=K)
        bits = to_bf16_bits(W).reshape(1, n * C)
        s, c, e, err = _run(bits, C, P, K, 4)
        planted = s.reshape(-1).astype(np.int64) == seeds.reshape(-1).astype(np.int64)
        _say(f"  planted seed recovered for {planted.sum()} of {n} blocks")
        assert planted.mean() >= 0.8
        assert np.array_equal(c.reshape(-1, P)[planted], coeffs.reshape(-1, P)[planted])
        assert np.array_equal(e.reshape(-1)[planted], exps.reshape(-1)[planted])
        Wb = _blocks(bf16_to_float64(bits), C)
        wn = np.sum(Wb ** 2, axis=1)
        dec = O.decode_rows(s.reshape(n, 1), c.reshape(n, 1, P), e.reshape(n, 1), C, C, P, K=K)
        assert np.all(np.abs(err - np.sum((Wb - dec) ** 2, axis=1)) <= SCORE_TOL * wn)
        # no worse than the planted record itself
        assert np.all(err <= np.sum((Wb - W.reshape(n, C)) ** 2, axis=1) + SCORE_TOL * wn)


@pytest.mark.parametrize("C,P,rows,cols", [(8, 3, 6, 8 * 9 + 3), (12, 4, 5, 12 * 7 + 4),
                                          (8, 3, 3, 5), (12, 4, 2, 12 * 341 + 4)])
def test_encode_ragged_columns(C, P, rows, cols):
    """cols not a multiple of C (4096 = 12*341 + 4 for the 3-bit Llama shapes): a row's
    last block holds its real weights followed by zeros and is searched as a full
    block, so the oracle's search runs on the same zero-padded block.  The records
    pack and decode at the real shape."""
    _say(f"encode ragged C={C} {rows}x{cols}")
    nb = -(-cols // C)
    bits = gen_bf16_weights(10, 1000 + cols, rows, cols)
    s, c, e, err = _run(bits, C, P)
    assert s.shape == (rows, nb) and c.shape == (rows, nb, P)
    padded = np.zeros((rows, nb * C), dtype=np.float64)
    padded[:, :cols] = bf16_to_float64(bits)
    Wb = _blocks(padded, C)
    k = Wb.shape[0]
    if k > 64:  # check the row ends and a sample of the rest against the search
        idx = np.unique(np.concatenate([np.arange(nb - 1, k, nb),
                                        np.random.default_rng(3).choice(k, 24, replace=False)]))
    else:
        idx = np.arange(k)
    _check_blocks(Wb[idx], s.reshape(k)[idx], c.reshape(k, P)[idx], e.reshape(k)[idx],
                  err.reshape(k)[idx], C, P, min_seed_match=0.8)
    S = _S()
    m = S.seedlm_pack(s.astype(np.uint16), c, e, rows, cols, C, P, 16)
    Wd = torch.empty((rows, cols), dtype=torch.float32, device=_dev())
    S.seedlm_decode(m, Wd)
    torch.cuda.synchronize()
    ref = O.decode_rows(s, c, e, cols, C, P)
    assert np.array_equal(Wd.cpu().numpy(), ref.astype(np.float32))
