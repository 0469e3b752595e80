"""bf16 <-> float64 by definition (oracle side).

bf16 is the upper 16 bits of an IEEE-754 binary32: 1 sign bit, 8 exponent
bits (bias 127), 7 stored fraction bits.  Rounding is round-to-nearest,
ties-to-even, applied once, directly from float64 (no float32 detour).

Test infrastructure only: imported by tests/ and bench.py's CPU leg, never by
the product path.
"""

from __future__ import annotations

import numpy as np

_EMIN = -126          # smallest normal exponent
_FRAC = 7             # stored fraction bits
_MAX_FINITE = (2.0 - 2.0 ** -_FRAC) * 2.0 ** 127


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def is_nonfinite_bits(bits: np.ndarray) -> np.ndarray:
    """True where the exponent field is all ones (Inf or NaN)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b & np.uint16(0x7F80)) == np.uint16(0x7F80)


def f64_to_bits(x) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest, ties to even.

    For |x| in binade [2^e, 2^(e+1)) the bf16 spacing is 2^(e-7); below the
    normal range the spacing stays 2^(-126-7).  Rounding x to the nearest
    multiple of that spacing (numpy.rint is ties-to-even) and converting the
    now exactly representable result to binary32 gives the pattern.  Results
    beyond the largest finite bf16 become +-Inf; NaN maps to 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    inf = np.isinf(x)
    ax = np.abs(np.where(nan | inf, 0.0, x))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    # log2 can be off by one ulp near powers of two: correct the binade.
    e = np.where(2.0 ** e > ax, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= ax, e + 1, e)
    q = 2.0 ** (np.maximum(e, _EMIN) - _FRAC)
    r = np.rint(np.where(nan | inf, 0.0, x) / q) * q
    over = (np.abs(r) > _MAX_FINITE) | inf
    r = np.where(over, np.copysign(np.inf, x), r)
    out[...] = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[nan] = np.uint16(0x7FC0)
    return out
