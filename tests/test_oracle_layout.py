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
    # one real row + 3 padding rows of one block each
    assert len(buf) == 16
    assert int.from_bytes(buf[0:4], "little") == int(g["word"][0], 16)
    for k in (1, 2, 3):
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
    rows, cols = 5, 320
    seeds, coeffs, exps = _unique_records(rows, 40, 3)
    buf = O.write_packed(seeds, coeffs, exps, rows, cols, 8, 3)
    assert len(buf) == 4 * 8 * 40

    def seed_at(k):
        return int.from_bytes(buf[4 * k:4 * k + 2], "little")

    # (r, b) -> word index, by hand from p*Mp*32 + (quad*Qp + q)*4 + r4
    cases = {(0, 0): 0, (3, 1): 7, (4, 0): 128, (2, 33): 262, (4, 39): 316, (1, 31): 125}
    for (r, b), k in cases.items():
        assert seed_at(k) == seeds[r, b], (r, b, k)
    # padding rows (r = 5..7) hold the word 0x00000001
    for r4 in (1, 2, 3):
        assert int.from_bytes(buf[4 * (128 + r4):4 * (128 + r4) + 4], "little") == 1
    assert O.padding_words_ok(buf, rows, cols, 8, 3)


def test_exponent_positions_worked_by_hand_3bit():
    # rows=5 -> Mp=8; cols=36 -> nb=3 (one panel of width 3); 24 words = 96 B;
    # the exponent array starts at byte 256 and holds (8/4)*3 = 6 uint16.
    rows, cols = 5, 36
    seeds, coeffs, exps = _unique_records(rows, 3, 4)
    buf = O.write_packed(seeds, coeffs, exps, rows, cols, 12, 4)
    assert len(buf) == 256 + 12
    # (r=4, b=2): quad 1, q 2 -> uint16 number 1*3 + 2 = 5, nibble 0
    v = int.from_bytes(buf[256 + 10:256 + 12], "little")
    assert (v & 0xF) == exps[4, 2] + 15 and (v >> 4) == 0
    # (r=1, b=0): quad 0, q 0 -> uint16 number 0, nibble 1
    v = int.from_bytes(buf[256:258], "little")
    assert ((v >> 4) & 0xF) == exps[1, 0] + 15
    # the word of (r=1, b=0) holds t3 in bits 28..31
    w = int.from_bytes(buf[4:8], "little")
    assert w & 0xFFFF == seeds[1, 0]


@pytest.mark.parametrize("C,P,rows,cols", [(8, 3, 7, 8 * 70), (12, 4, 6, 12 * 33 + 5), (8, 3, 4, 3)])
def test_round_trip(C, P, rows, cols):
    rng = np.random.default_rng(rows * cols)
    nb = -(-cols // C)
    seeds = rng.integers(1, 65536, (rows, nb)).astype(np.uint16)
    coeffs = rng.integers(-8, 8, (rows, nb, P)).astype(np.int8)
    exps = rng.integers(-15, 1, (rows, nb)).astype(np.int8)
    buf = O.write_packed(seeds, coeffs, exps, rows, cols, C, P)
    assert len(buf) == O.packed_size(rows, cols, C, P)
    s, c, e = O.read_packed(buf, rows, cols, C, P)
    assert (s == seeds).all() and (c == coeffs).all() and (e == exps).all()


def test_writer_rejects_bad_records():
    seeds = np.ones((1, 1), np.uint16)
    with pytest.raises(ValueError):
        O.write_packed(seeds * 0, np.zeros((1, 1, 3), np.int8), np.zeros((1, 1), np.int8), 1, 8, 8, 3)
    with pytest.raises(ValueError):
        O.write_packed(seeds, np.zeros((1, 1, 3), np.int8), np.zeros((1, 1), np.int8), 1, 8, 8, 4)
