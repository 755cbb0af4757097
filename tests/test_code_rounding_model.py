"""CPU model of the row-streaming kernel's code rounding, checked against the
oracle's quantizer on every 16-bit value of a row.

The kernel never divides per element.  With rinv = 1/s it forms two fp32
products that bracket the IEEE quotient, y * rinv * (1 + 2^-21) and
y * rinv * (1 - 2^-21), each rounded to an integer by one fused
multiply-add with 1.5 * 2^23.  Where the two integers agree they are
round-half-even(fl(y / s)).  Where they differ the quotient is within
2^-20 of a half-integer h = k + 1/2, which for 16-bit y and absmax a only
happens at an exact tie 7 y = h a; every element of the row that ties at h
has the same |y|, so one IEEE division per h (seven per row, one per lane)
gives the outcome for all of them.  The model below takes exactly these
steps in fp32 (numpy's float32 arithmetic is IEEE round-to-nearest-even;
the fused multiply-add is exact because the fp64 product of a 16-bit value
and an fp32 value is exact) and must reproduce the oracle's codes for
every y with |y| <= a, for absmax values spread over the whole range:
subnormal, clamped scale (a / 7 below 2^-126), around 2^64 (where the tie
values are formed at a 2^-64 scale) and the largest finite value.

Rows whose absmax has an integer significand that 7 does not divide can only
tie at y = a / 2 (7 y = (k + 1/2) a needs 7 | 2k + 1): there the kernel takes
one fma per element with the multiplier that rounds that tie the quantizer's
way, and that single rounding must reproduce the oracle as well."""
import numpy as np
import pytest

import oracle

F32 = np.float32


def _mask_bits(a, s, clamped, dtype):
    """Bit k (k = 0..6): a tie at h = k + 1/2 rounds away from zero."""
    if clamped:
        return 0x2A
    b = 0
    big = a > F32(2.0 ** 64)
    ah = F32(a * F32(2.0 ** -64)) if big else a
    for k in range(7):
        h = F32(k + 0.5)
        yh = F32(F32(h * ah) / F32(7.0))
        if big:
            yh = F32(yh * F32(2.0 ** 64))
        qh = F32(yh / s)
        if np.rint(qh) > h:
            b |= 1 << k
    return b


def _bitrev32(v):
    return int(f"{v & 0xFFFFFFFF:032b}"[::-1], 2)


def model_codes(y, a, dtype):
    """Codes of the values y (fp32 array) in a row whose absmax is a."""
    a = F32(a)
    s = F32(a / F32(7.0))
    if s < F32(2.0 ** -126):
        s = F32(2.0 ** -126)
    rinv = F32(F32(1.0) / s)
    rh = F32(rinv * F32(1.0 + 2.0 ** -21))
    rl = F32(rinv * F32(1.0 - 2.0 ** -21))
    u = np.rint(y.astype(np.float64) * np.float64(rh)).astype(np.int64)
    d = np.rint(y.astype(np.float64) * np.float64(rl)).astype(np.int64)
    b = _mask_bits(a, s, s == F32(2.0 ** -126), dtype)
    mask = (b | (_bitrev32(b) << 1)) & 0xFFFFFFFF
    up = (mask >> (d & 31)) & 1
    code = d + up * (u - d)
    return code.astype(np.int8), int((u != d).sum()), int(((u != d) & (up == 1)).sum())


def significand(ap, dtype):
    """Integer significand of a positive finite 16-bit pattern."""
    if dtype == "bf16":
        return (ap & 0x7F) | (0x80 if (ap >> 7) & 0xFF else 0)
    return (ap & 0x3FF) | (0x400 if (ap >> 10) & 0x1F else 0)


def model_codes_single(y, a, dtype):
    """Codes from one fma per element, for rows whose absmax significand 7
    does not divide: the multiplier that takes the tie y = a / 2 (k = 3) the
    quantizer's way (bit 3 of the tie table)."""
    a = F32(a)
    s = F32(a / F32(7.0))
    assert s >= F32(2.0 ** -126)
    rinv = F32(F32(1.0) / s)
    rh = F32(rinv * F32(1.0 + 2.0 ** -21))
    rl = F32(rinv * F32(1.0 - 2.0 ** -21))
    r1 = rh if _mask_bits(a, s, False, dtype) & 8 else rl
    return np.rint(y.astype(np.float64) * np.float64(r1)).astype(np.int64).astype(np.int8)


def _patterns(dtype, rng):
    """Positive finite absmax bit patterns covering the range."""
    if dtype == "bf16":
        fixed = [0x0001, 0x0002, 0x007F, 0x0080, 0x0081, 0x00E0, 0x0380, 0x03B0, 0x03C0, 0x03FF,
                 0x0400, 0x3F80, 0x40E0, 0x4100, 0x5F7F, 0x5F80, 0x5F81, 0x5FD0, 0x7F7F, 0x7F00]
        top = 0x7F7F
    else:
        fixed = [0x0001, 0x0002, 0x0007, 0x000E, 0x03FF, 0x0400, 0x0401, 0x3C00, 0x4700, 0x4B00,
                 0x4B80, 0x7BFF, 0x7800]
        top = 0x7BFF
    extra = rng.integers(1, top + 1, size=60).tolist()
    return sorted(set(fixed + extra))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_bracket_and_tie_table_reproduce_the_quantizer(dtype):
    rng = np.random.default_rng(17)
    ties = ups = single = table = 0
    for ap in _patterns(dtype, rng):
        pos = np.arange(0, ap + 1, dtype=np.uint32)
        bits = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
        vals = oracle.decode(dtype, bits)
        a = float(oracle.decode(dtype, np.array([ap], np.uint16))[0])
        ref_codes, ref_s = oracle.quantize(bits[None, :], dtype)
        got, nt, nu = model_codes(vals.astype(np.float32), a, dtype)
        bad = np.flatnonzero(got != ref_codes[0])
        assert bad.size == 0, (hex(ap), [(hex(int(bits[i])), int(got[i]), int(ref_codes[0][i])) for i in bad[:5]])
        ties += nt
        ups += nu
        if significand(ap, dtype) % 7 and F32(F32(a) / F32(7.0)) >= F32(2.0 ** -126):
            one = model_codes_single(vals.astype(np.float32), a, dtype)
            bad = np.flatnonzero(one != ref_codes[0])
            assert bad.size == 0, ("single", hex(ap), [(hex(int(bits[i])), int(one[i]), int(ref_codes[0][i]))
                                                        for i in bad[:5]])
            single += 1
        else:
            table += 1
    # both outcomes of a tie occur (a rule that always rounds half to even,
    # or always away from zero, would fail above)
    assert ties > 0 and 0 < ups < ties, (ties, ups)
    # both paths of the kernel are exercised
    assert single > 10 and table > 3, (single, table)
