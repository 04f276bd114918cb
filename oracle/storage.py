"""Storage formats seen by the oracle (test infrastructure only).

The oracle computes in float64. Inputs arrive as their stored values (float32
arrays, or bf16 as raw uint16 bit patterns) and outputs leave rounded to the
parameter's storage format with round-to-nearest-even, as the speedtronic
"v2 optimizers" page's "Muon update" section implies for momentum kept in FP32
"independently of parameter precision" and parameters kept in their own dtype.

bf16 here is the 16-bit format with 8 exponent bits and 8 significant bits
(7 stored): the top half of an IEEE binary32 pattern.
"""
import numpy as np


def decode(arr, dtype: str) -> np.ndarray:
    """Stored values -> float64. ``dtype`` is "f32" or "bf16" (uint16 bits)."""
    a = np.asarray(arr)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 values must be given as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_f32(x) -> np.ndarray:
    """float64 -> nearest binary32 (numpy's conversion rounds to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_bf16_bits(x) -> np.ndarray:
    """float64 -> bf16 bit patterns, rounded once, to nearest, ties to even.

    A finite value x = f * 2**e with 0.5 <= |f| < 1 keeps 8 significant bits:
    the quantum is 2**(e - 8), floored at the smallest subnormal step 2**-133.
    np.rint rounds halves to even. The rounded value is exact in binary32, so
    its top 16 bits are the bf16 pattern. NaN maps to the quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(x / q) * q
    r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, r), r)
    bits = r.astype(np.float32).view(np.uint32) >> np.uint32(16)
    out[...] = bits.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def round_to(x, dtype: str) -> np.ndarray:
    """float64 -> storage representation (float32 array or bf16 uint16 bits)."""
    if dtype == "f32":
        return round_f32(x)
    if dtype == "bf16":
        return round_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")
