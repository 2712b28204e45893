"""Pins for the oracle's LFSR: invariants that a primitive degree-16 polynomial
fixes, and states worked out by hand (tests/golden/block_seed1.txt)."""
import numpy as np
import pytest

from oracle import seedlm_oracle as O


def test_period_is_full_and_visits_every_nonzero_state():
    # A primitive polynomial of degree 16 gives a maximal-length sequence:
    # period 2^16 - 1, every nonzero state exactly once.
    z = 1
    seen = bytearray(1 << 16)
    for n in range(1, 70000):
        seen[z] += 1
        z = O.lfsr_step(z)
        if z == 1:
            break
    assert n == 65535
    assert seen[0] == 0
    assert all(seen[s] == 1 for s in range(1, 1 << 16))


def test_sum_of_centered_states_over_a_period_is_zero():
    # sum_{z=1}^{65535} (z - 2^15) = 65535*65536/2 - 65535*32768 = 0
    states = O.lfsr_states(12345, 65535)
    assert sum(z - 32768 for z in states) == 0


def test_zero_state_is_rejected_and_fixed_point():
    assert O.lfsr_step(0) == 0  # the all-zero state locks: why seed 0 is invalid
    import pytest
    with pytest.raises(ValueError):
        O.lfsr_states(0, 4)
    with pytest.raises(ValueError):
        O.lfsr_states(65536, 4)


def test_hand_worked_states(golden):
    g = golden("block_seed1.txt")
    seed = int(g["seed"][0])
    want = [int(v) for v in g["states"]]
    assert O.lfsr_states(seed, len(want)) == want


def test_single_bit_seeds_fall_one_place_per_step():
    # While the set bit is above bit 5 the feedback (bits 0,2,3,5) is zero.
    for k in range(6, 16):
        assert O.lfsr_step(1 << k) == 1 << (k - 1)
    # Bits 0, 2, 3, 5 each feed back into bit 15.
    for k in (0, 2, 3, 5):
        assert O.lfsr_step(1 << k) == (1 << 15) | ((1 << k) >> 1)
    for k in (1, 4):
        assert O.lfsr_step(1 << k) == 1 << (k - 1)


def test_states_form_a_sliding_window_of_one_bit_stream():
    # Fibonacci right-shift form: z_{n+1} keeps bits 1..15 of z_n as bits 0..14.
    states = O.lfsr_states(0xACE1, 200)
    for a, b in zip(states, states[1:]):
        assert (b & 0x7FFF) == (a >> 1)


def test_gf2_linearity_of_the_state_sequence():
    # An LFSR is linear over GF(2): seq(s1 ^ s2) = seq(s1) ^ seq(s2).
    rng = np.random.default_rng(7)
    for _ in range(20):
        s1, s2 = (int(v) for v in rng.integers(1, 65536, 2))
        if s1 == s2:
            continue
        a = O.lfsr_states(s1, 48)
        b = O.lfsr_states(s2, 48)
        c = O.lfsr_states(s1 ^ s2, 48)
        assert [x ^ y for x, y in zip(a, b)] == c


# Other seed widths of the design-space study: each LFSR must be maximal-length.
@pytest.mark.parametrize("K", [12, 20])
def test_other_seed_widths_have_full_period(K):
    n = (1 << K) - 1
    seen = np.zeros(1 << K, dtype=bool)
    z, total = 1, 0
    for _ in range(n):
        assert not seen[z]
        seen[z] = True
        total += z - (1 << (K - 1))
        z = O.lfsr_step(z, K)
    assert z == 1                      # back at the seed after exactly 2^K - 1 steps
    assert seen[1:].all() and not seen[0]
    assert total == 0                  # the values (z - 2^(K-1)) sum to zero over a period


def test_other_seed_widths_first_states_by_hand():
    # K = 12, feedback bits 0,1,4,6 of z enter at bit 11.  From z = 1: bit 0 is
    # set, so f = 1 and z1 = 0 | 1 << 11 = 2048; then 2048 has none of bits
    # 0,1,4,6 set: z2 = 1024, z3 = 512, z4 = 256, z5 = 128.
    assert O.lfsr_states(1, 6, 12) == [1, 2048, 1024, 512, 256, 128]
    # K = 20, feedback bits 0,3 enter at bit 19: z1 = 2^19, then halving.
    assert O.lfsr_states(1, 6, 20) == [1, 524288, 262144, 131072, 65536, 32768]
    with pytest.raises(ValueError):
        O.lfsr_states(4096, 2, 12)
