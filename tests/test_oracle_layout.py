"""Pins for the oracle's packed-layout reader and writer: the hand-packed word
of the golden block, word/exponent positions worked out by hand for a small
ragged case, round trips, and padding rows."""
import numpy as np
import pytest

from oracle import seedlm_oracle as O


def test_golden_word(golden):
    g = golden("block_seed1.txt")
    seeds = np.array([[int(g["seed"][0])]], np.uint16)
    coeffs = np.array([[[int(v) for v in g["t"]]]], np.int8)
    exps = np.array([[int(g["e"][0])]], np.int8)
    buf = O.write_packed(seeds, coeffs, exps, 1, 8, 8, 3)
    # one row, one block; rows are padded to 8 and the panel to 4 slots
    assert len(buf) == 4 * 8 * 4
    assert int.from_bytes(buf[0:4], "little") == int(g["word"][0], 16)
    for k in range(1, 32):
        assert int.from_bytes(buf[4 * k:4 * k + 4], "little") == 1
    s, c, e = O.read_packed(buf, 1, 8, 8, 3)
    assert (s == seeds).all() and (c == coeffs).all() and (e == exps).all()


def _unique_records(rows, nb, P):
    seeds = (np.arange(rows * nb).reshape(rows, nb) + 1).astype(np.uint16)
    coeffs = np.zeros((rows, nb, P), np.int8)
    coeffs[..., 0] = (np.arange(rows)[:, None] % 16) - 8
    exps = -(np.arange(nb)[None, :] % 16 + 0 * np.arange(rows)[:, None]).astype(np.int8)
    return seeds, coeffs, exps


def test_word_positions_worked_by_hand_4bit():
    # rows=5 -> Mp=8; cols=320 -> nb=40: panel 0 has 32 blocks, panel 1 has 8.
    # word(r, b) = p*8*32 + r*Wp' + 4*(q//4) + ((q - r) mod 4)
    rows, cols = 5, 320
    seeds, coeffs, exps = _unique_records(rows, 40, 3)
    buf = O.write_packed(seeds, coeffs, exps, rows, cols, 8, 3)
    assert len(buf) == 4 * (8 * 32 + 8 * 8)

    def seed_at(k):
        return int.from_bytes(buf[4 * k:4 * k + 2], "little")

    cases = {(0, 0): 0, (3, 1): 98, (4, 0): 128, (2, 33): 275, (4, 39): 295, (1, 31): 62}
    for (r, b), k in cases.items():
        assert seed_at(k) == seeds[r, b], (r, b, k)
    # padding rows 5..7 of panel 0 start at word 5*32 = 160
    assert all(int.from_bytes(buf[4 * k:4 * k + 4], "little") == 1 for k in range(160, 256))
    assert O.padding_words_ok(buf, rows, cols, 8, 3)


def test_narrow_last_panel_is_padded_to_four_slots():
    # rows = 3 -> Mp = 8; cols = 8*37 -> nb = 37: panel 1 has 5 blocks, padded to 8 slots.
    rows, cols = 3, 8 * 37
    seeds, coeffs, exps = _unique_records(rows, 37, 3)
    buf = O.write_packed(seeds, coeffs, exps, rows, cols, 8, 3)
    assert len(buf) == 4 * (8 * 32 + 8 * 8)
    assert O.padding_words_ok(buf, rows, cols, 8, 3)
    # row 2, block 36 (panel 1, q=4): 256 + 2*8 + 4 + ((4-2) mod 4) = 278
    assert int.from_bytes(buf[4 * 278:4 * 278 + 2], "little") == seeds[2, 36]
    # row 1, slot 6 is padding: position 4 + ((6-1) mod 4) = 5 -> word 256 + 8 + 5 = 269
    assert int.from_bytes(buf[4 * 269:4 * 269 + 4], "little") == 1


def test_exponent_positions_worked_by_hand_3bit():
    # rows=5 -> Mp=8; cols=36 -> nb=3: one panel, width 3 padded to 4; 32 words
    # = 128 B; the exponent array starts at byte 256 and holds 8 uint16 (one per row).
    rows, cols = 5, 36
    seeds, coeffs, exps = _unique_records(rows, 3, 4)
    buf = O.write_packed(seeds, coeffs, exps, rows, cols, 12, 4)
    assert len(buf) == 256 + 16
    assert O.padding_words_ok(buf, rows, cols, 12, 4)
    # (r=4, b=2): word 4*4 + ((2-4) mod 4) = 18; exponent uint16 number 4, nibble 2
    assert int.from_bytes(buf[4 * 18:4 * 18 + 2], "little") == seeds[4, 2]
    v = int.from_bytes(buf[256 + 8:256 + 10], "little")
    assert ((v >> 8) & 0xF) == exps[4, 2] + 15
    # (r=1, b=0): word 4 + ((0-1) mod 4) = 7; exponent uint16 number 1, nibble 3
    assert int.from_bytes(buf[28:30], "little") == seeds[1, 0]
    v = int.from_bytes(buf[256 + 2:256 + 4], "little")
    assert ((v >> 12) & 0xF) == exps[1, 0] + 15
    # (r=1, pad slot q=3): position (3-1) mod 4 = 2 -> word 6, pad word with g nibble 0
    assert int.from_bytes(buf[24:28], "little") == 1
    assert ((v >> 8) & 0xF) == 0


def test_word_and_exponent_positions_worked_by_hand_3bit_panels_of_16():
    # rows=3 -> Mp=8; cols=12*20 -> nb=20: C=12 panels hold 16 blocks, so panel
    # 0 has 16 blocks (rows of 16 words) and panel 1 has 4 (rows of 4 words,
    # starting at word 8*16 = 128).  160 words = 640 B; exponents start at byte
    # 768 and hold 160/4 = 40 uint16 (panel 0: 8 rows x 4, panel 1 from 32).
    rows, cols = 3, 12 * 20
    seeds, coeffs, exps = _unique_records(rows, 20, 4)
    buf = O.write_packed(seeds, coeffs, exps, rows, cols, 12, 4)
    assert len(buf) == 768 + 80
    assert O.padding_words_ok(buf, rows, cols, 12, 4)

    def seed_at(k):
        return int.from_bytes(buf[4 * k:4 * k + 2], "little")

    def nibble_at(k, j):
        return (int.from_bytes(buf[768 + 2 * k:768 + 2 * k + 2], "little") >> (4 * j)) & 0xF

    # (r=2, b=17): panel 1, q=1: 128 + 2*4 + ((1-2) mod 4 = 3) = 139; exps 32 + 2 = 34, nibble 3
    assert seed_at(139) == seeds[2, 17] and nibble_at(34, 3) == exps[2, 17] + 15
    # (r=1, b=14): panel 0, q=14: 16 + 12 + ((14-1) mod 4 = 1) = 29; exps 4 + 3 = 7, nibble 1
    assert seed_at(29) == seeds[1, 14] and nibble_at(7, 1) == exps[1, 14] + 15
    # (r=0, b=19): panel 1, q=3: 128 + 3 = 131; exps 32, nibble 3
    assert seed_at(131) == seeds[0, 19] and nibble_at(32, 3) == exps[0, 19] + 15
    # the first padding row of panel 1 (r=3) starts at word 128 + 12 = 140
    assert all(int.from_bytes(buf[4 * k:4 * k + 4], "little") == 1 for k in range(140, 160))


def test_words_of_the_other_formats_worked_by_hand():
    # (8,4,16), 3-bit coefficients: seed 0x1234, t = (1, -2, 3, -4), e = -6:
    # 0x1234 | 1<<16 | 6<<19 | 3<<22 | 4<<25 | 9<<28 = 0x98F11234
    buf = O.write_packed(np.array([[0x1234]], np.uint16), np.array([[[1, -2, 3, -4]]], np.int8),
                         np.array([[-6]], np.int8), 1, 8, 8, 4, K=16)
    assert len(buf) == 4 * 8 * 4
    assert int.from_bytes(buf[0:4], "little") == 0x98F11234
    # (12,3,20): seed 0xABCDE, t = (7, -8, -1), e = -15:
    # 0xABCDE | 7<<20 | 8<<24 | 15<<28 = 0xF87ABCDE, exponent nibble 0
    buf = O.write_packed(np.array([[0xABCDE]], np.uint32), np.array([[[7, -8, -1]]], np.int8),
                         np.array([[-15]], np.int8), 1, 12, 12, 3, K=20)
    assert len(buf) == 256 + 16
    assert int.from_bytes(buf[0:4], "little") == 0xF87ABCDE
    assert buf[256] & 0xF == 0
    # 3-bit coefficients outside [-4, 3] are rejected
    with pytest.raises(ValueError):
        O.write_packed(np.array([[1]], np.uint16), np.array([[[4, 0, 0, 0]]], np.int8),
                       np.array([[0]], np.int8), 1, 8, 8, 4, K=16)


@pytest.mark.parametrize("C,P,K,rows,cols", [(8, 3, 16, 7, 8 * 70), (12, 4, 16, 6, 12 * 33 + 5),
                                             (8, 3, 16, 4, 3), (8, 4, 16, 5, 8 * 40 + 3),
                                             (12, 3, 20, 9, 12 * 37 + 8)])
def test_round_trip(C, P, K, rows, cols):
    rng = np.random.default_rng(rows * cols)
    nb = -(-cols // C)
    Q = O.PACKED_FORMATS[(C, P, K)]
    seeds = rng.integers(1, 1 << K, (rows, nb)).astype(np.uint16 if K <= 16 else np.uint32)
    coeffs = rng.integers(-(1 << (Q - 1)), 1 << (Q - 1), (rows, nb, P)).astype(np.int8)
    exps = rng.integers(-15, 1, (rows, nb)).astype(np.int8)
    buf = O.write_packed(seeds, coeffs, exps, rows, cols, C, P, K=K)
    assert len(buf) == O.packed_size(rows, cols, C, P)
    assert O.padding_words_ok(buf, rows, cols, C, P)
    s, c, e = O.read_packed(buf, rows, cols, C, P, K=K)
    assert (s == seeds).all() and (c == coeffs).all() and (e == exps).all()


def test_writer_rejects_bad_records():
    seeds = np.ones((1, 1), np.uint16)
    with pytest.raises(ValueError):
        O.write_packed(seeds * 0, np.zeros((1, 1, 3), np.int8), np.zeros((1, 1), np.int8), 1, 8, 8, 3)
    with pytest.raises(ValueError):
        O.write_packed(seeds, np.zeros((1, 1, 3), np.int8), np.zeros((1, 1), np.int8), 1, 8, 8, 4)
