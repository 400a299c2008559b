"""bf16 <-> float64 for the oracle (test infrastructure only).

bf16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent bits,
7 stored significand bits.  Values are carried as uint16 bit patterns.
"""
import numpy as np


def to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16 array) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even; returns float64.

    Written from the definition: with E = floor(log2|x|) the bf16 spacing is
    2^(max(E, -126) - 7) (8 significant bits for normal numbers, fixed spacing
    2^-133 in the subnormal range), and x is rounded to the nearest multiple of
    that spacing with ties to the even multiple (numpy.rint).  Magnitudes above
    the largest finite bf16 become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])                    # |x| = f * 2^e, f in [0.5, 1)
    E = e.astype(np.int64) - 1                # floor(log2|x|)
    q = np.ldexp(1.0, np.maximum(E, -126) - 7)
    r = np.rint(x[nz] / q) * q                # division by a power of two is exact
    big = np.abs(r) > 3.3895313892515355e38   # max finite bf16
    r[big] = np.copysign(np.inf, r[big])
    out[nz] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def to_bits(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of float64 values that are already bf16 values."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
