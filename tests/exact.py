"""Exact-rational helpers for the oracle pins (test code, independent of the
oracle's C implementation)."""
from __future__ import annotations

import bisect
import functools
from fractions import Fraction

import numpy as np


@functools.lru_cache(maxsize=None)
def finite_values(fmt: str):
    """All finite values of a 16-bit format as sorted exact Fractions, with the
    parity of each value's last significand bit (for ties to even)."""
    vals = {}
    for b in range(1 << 16):
        if fmt == "f16":
            s, e, m = b >> 15, (b >> 10) & 31, b & 1023
            if e == 31:
                continue
            v = Fraction(m, 1 << 24) if e == 0 else Fraction(1024 + m, 1) * Fraction(2) ** (e - 25)
            even = (m & 1) == 0
        else:  # bf16
            s, e, m = b >> 15, (b >> 7) & 255, b & 127
            if e == 255:
                continue
            v = Fraction(m) * Fraction(2) ** (-133) if e == 0 else Fraction(128 + m) * Fraction(2) ** (e - 134)
            even = (m & 1) == 0
        if s:
            v = -v
        if v not in vals or even:
            vals[v] = even
    keys = sorted(vals)
    return keys, [vals[k] for k in keys]


def round_exact(v: Fraction, fmt: str) -> float:
    """Nearest value of fmt to the exact rational v, ties to the even
    significand; beyond the largest finite value by at least half an ulp of the
    next binade -> +-inf."""
    keys, even = finite_values(fmt)
    big = keys[-1]
    if fmt == "f16":
        limit = Fraction(65520)
    else:
        limit = Fraction(2) ** 128 - Fraction(2) ** 119
    if v >= limit:
        return float("inf")
    if v <= -limit:
        return float("-inf")
    i = bisect.bisect_left(keys, v)
    if i < len(keys) and keys[i] == v:
        return float(v)
    lo, hi = keys[i - 1], keys[i]
    if v - lo < hi - v:
        return float(lo)
    if hi - v < v - lo:
        return float(hi)
    return float(lo) if even[i - 1] else float(hi)


def round_exact_f32(v: Fraction) -> float:
    """Nearest binary32 to an exact rational (ties to even), via the exact
    neighbours of the float64 nearest to v."""
    f = np.float32(float(v))  # candidate within one ulp
    cands = {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))}
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - v)
        bits = np.array([c], dtype=np.float32).view(np.uint32)[0]
        key = (d, int(bits) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return float(best[1])


def rne(v: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even (Python's round)."""
    return round(v)
