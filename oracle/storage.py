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


# -- dew.training.optim "stochastic_round_bf16" -------------------------------
# The pages ask for a counter-based hash of the seed and each element's flat
# index and name none. The one used is SplitMix64 (Steele, Lea and Flood, "Fast
# splittable pseudorandom number generators", OOPSLA 2014): state advanced by
# the golden-ratio increment, output function mix64 below.
SPLITMIX_GAMMA = 0x9E3779B97F4A7C15
_M64 = (1 << 64) - 1


def splitmix64_mix(z):
    """SplitMix64's output function on uint64 values (array or int)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):   # arithmetic modulo 2^64 is the definition
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def sr_key(seed, step, leaf, moment):
    """Key of one (step, tensor, moment) stream: mix(seed ^ mix((step << 32) +
    (leaf << 1) + moment)), all modulo 2^64."""
    c = ((int(step) << 32) + (int(leaf) << 1) + int(moment)) & _M64
    return int(splitmix64_mix(np.uint64(int(seed) & _M64) ^ splitmix64_mix(np.uint64(c))))


def stochastic_round_bf16_bits(x32, key, index0=0):
    """binary32 values -> bf16 bit patterns: add 16 uniform bits below the kept
    mantissa and truncate, so a value rounds up with the probability of its
    distance from the lower neighbour; NaN stays NaN (a quiet NaN). The bits
    of element i (flat index index0 + i) are the top 16 of SplitMix64's output
    at state key + (index0 + i + 1) * gamma."""
    x32 = np.ascontiguousarray(np.asarray(x32, dtype=np.float32))
    u = x32.reshape(-1).view(np.uint32).astype(np.uint64)
    idx = np.arange(u.size, dtype=np.uint64) + np.uint64(int(index0) + 1)
    with np.errstate(over="ignore"):
        state = np.uint64(int(key) & _M64) + idx * np.uint64(SPLITMIX_GAMMA)
    r = splitmix64_mix(state) >> np.uint64(48)
    out = ((u + r) >> np.uint64(16)).astype(np.uint16)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return out.reshape(x32.shape)
