"""Pins for the host-side bf6 (e3m2) decoder the FP6 GEMM tests read GPU
output with: closed-form facts of the format (largest value 28, smallest
normal 1/4, smallest subnormal 1/16, every value a multiple of 1/16, sign
symmetry), the exact encodings of the integers -8..8, and the block bit
layout against a hand-built block."""
import numpy as np

from tests.bf6 import TABLE, decode_blocks, value


def test_value_set():
    pos = TABLE[:32]
    assert pos.max() == 28.0 and sorted(pos)[1] == 0.0625
    assert min(v for v in pos if v >= 0.25) == 0.25 and value(0x04) == 0.25
    assert np.all(np.mod(pos * 16, 1) == 0)                  # multiples of 1/16
    assert np.all(TABLE[32:] == -TABLE[:32])                  # sign bit 5
    assert len(set(pos.tolist())) == 32                       # no duplicates, no specials
    assert np.all(np.diff(pos) > 0)                           # monotone in the pattern


def test_integers_are_exact():
    enc = {0: 0x00, 1: 0x0C, 2: 0x10, 3: 0x12, 4: 0x14, 5: 0x15, 6: 0x16, 7: 0x17, 8: 0x18}
    for v, p in enc.items():
        assert value(p) == v and value(p | 0x20) == -v
    ints = [v for v in TABLE if v == int(v) and abs(v) <= 8]
    assert sorted(set(ints)) == list(range(-8, 9))


def test_block_layout():
    # value e in bits 6e .. 6e+5: build a block of the patterns e (0..31)
    bits = 0
    for e in range(32):
        bits |= e << (6 * e)
    blk = np.array([(bits >> (8 * b)) & 0xFF for b in range(24)] + [0] * 8, np.uint8)[None, :]
    vals, pad = decode_blocks(blk)
    assert np.array_equal(vals[0], TABLE[:32]) and not pad.any()
