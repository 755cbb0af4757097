"""bf6 (e3m2) blocks, decoded on the host from the format's definition: sign
bit 5, exponent bits 4-2 with bias 3, mantissa bits 1-0; exponent 0 is
subnormal (m / 4 * 2^-2); no infinities or NaN.  A block holds 32 values in
24 bytes (value e in bits 6e .. 6e+5 of the little-endian 192-bit block)
followed by 8 unused bytes."""
import numpy as np


def value(p: int) -> float:
    s = -1.0 if p & 0x20 else 1.0
    e = (p >> 2) & 7
    m = p & 3
    if e == 0:
        return s * (m / 4.0) * 2.0 ** -2
    return s * (1.0 + m / 4.0) * 2.0 ** (e - 3)


TABLE = np.array([value(p) for p in range(64)])


def decode_blocks(buf: np.ndarray) -> tuple:
    """(rows, K) uint8 bf6 blocks -> (values (rows, K) float64, pad bytes)."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    rows, K = buf.shape
    blk = buf.reshape(rows, K // 32, 32)
    payload = blk[:, :, :24].astype(np.uint64)
    # 192-bit little-endian integer per block, as three 64-bit words
    words = [np.zeros(payload.shape[:2], np.uint64) for _ in range(3)]
    for byte in range(24):
        words[byte // 8] |= payload[:, :, byte] << np.uint64(8 * (byte % 8))
    vals = np.empty((rows, K // 32, 32), np.float64)
    for e in range(32):
        bit = 6 * e
        w, o = bit // 64, bit % 64
        p = (words[w] >> np.uint64(o)) & np.uint64(0x3F)
        if o > 58:
            p |= (words[w + 1] << np.uint64(64 - o)) & np.uint64(0x3F)
        vals[:, :, e] = TABLE[p.astype(np.int64)]
    return vals.reshape(rows, K), blk[:, :, 24:]
