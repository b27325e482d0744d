"""Exact-arithmetic helpers used only by the oracle pins.

They are written independently of the oracle: rational arithmetic with
``fractions.Fraction`` and rounding by picking the nearest float32 candidate.
"""
from fractions import Fraction

import numpy as np


def bf16_value(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern, decoded by IEEE field rules."""
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    assert e != 0xFF
    if e == 0:
        return s * Fraction(f, 1 << 7) * Fraction(1, 1 << 126)
    v = Fraction(128 + f, 128)
    return s * (v * (Fraction(2) ** (e - 127)))


def nearest_f32(v: Fraction) -> np.float32:
    """float32 nearest to the rational ``v`` (ties to even), by candidate search."""
    if v == 0:
        return np.float32(0.0)
    c = np.float32(float(v))          # float(Fraction) is correctly rounded to f64
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    cands = [x for x in cands if np.isfinite(x)]
    best = None
    for x in cands:
        d = abs(Fraction(float(x)) - v)
        key = (d, int(np.array(x, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, x)
    return np.float32(best[1])


def unpack_nibble(words, i, k):
    return (int(words[i, k // 8]) >> (4 * (k % 8))) & 0xF
