"""Small numpy helpers shared by the tests (bit patterns, tolerance checks)."""
from fractions import Fraction

import numpy as np


def f32_to_bf16_bits(v) -> np.ndarray:
    """bf16 bit patterns of fp32 values, round to nearest even."""
    u = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    u = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def random_bf16(rng, shape, std=1.0) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(std))


def exact_dot(a_bits, b_bits) -> Fraction:
    """The exact rational value of sum_i a_i * b_i for bf16 bit patterns."""
    a = bf16_bits_to_f64(a_bits)
    b = bf16_bits_to_f64(b_bits)
    return sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, b)), Fraction(0))


def is_rne_f32(value: Fraction, f: np.float32) -> bool:
    """True when f is the binary32 value nearest to `value`, ties to an even significand."""
    f = np.float32(f)
    if not np.isfinite(f):
        return False
    lo = np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(f, np.float32(np.inf))
    d = abs(value - Fraction(float(f)))
    dlo = abs(value - Fraction(float(lo))) if np.isfinite(lo) else None
    dhi = abs(value - Fraction(float(hi))) if np.isfinite(hi) else None
    for dn in (dlo, dhi):
        if dn is None:
            continue
        if dn < d:
            return False
        if dn == d and (int(np.array(f).view(np.uint32)) & 1):
            return False
    return True


def allclose_report(got, ref, atol, rtol):
    """Elementwise |got - ref| <= atol + rtol*|ref|; returns (ok, worst excess, index)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    lim = atol + rtol * np.abs(ref)
    excess = err - lim
    i = int(np.argmax(excess)) if excess.size else 0
    return bool((excess <= 0).all()), float(excess.ravel()[i]) if excess.size else 0.0, i
