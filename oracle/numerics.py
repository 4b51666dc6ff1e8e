"""Exact decoding and rounding of the KV storage types, in float64.

TEST INFRASTRUCTURE (see the package docstring).

bfloat16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits and
7 stored fraction bits. Decoding is exact (bits << 16 reinterpreted as
binary32, then widened). Rounding a float64 to bfloat16 is done in one step,
round to nearest with ties to even, with no intermediate binary32 rounding
(two roundings can differ from one).
"""
import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")   # largest finite bfloat16


def decode_bf16(bits):
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    For |x| in the normal range the spacing of bfloat16 values around x is
    2^(e-8), where x = f * 2^e with f in [0.5, 1); below 2^-126 the spacing is
    the subnormal step 2^-133. Dividing by that spacing (exact: a power of
    two), rounding to the nearest integer with ties to even (numpy.rint), and
    scaling back gives the correctly rounded value. Values whose rounded
    magnitude exceeds the largest finite bfloat16 become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)
    qexp = np.where(e - 1 < -126, -133, e - 8).astype(np.int64)
    q = np.ldexp(np.ones_like(ax), qexp)
    r = np.rint(ax / q) * q
    r = np.where(ax == 0.0, 0.0, r)
    r = np.where(r > BF16_MAX, np.inf, r)
    r = np.where(np.isnan(x), np.nan, r)
    return np.copysign(r, x)


def bf16_bits_of(x):
    """bfloat16 bit patterns of float64 values that are already bfloat16 values."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_to_dtype(x, dtype):
    """Round float64 values to the KV storage type ('bf16' or 'f32'), ties to even."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        # numpy's float64 -> float32 conversion is the IEEE conversion
        # (round to nearest, ties to even).
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def decode(arr, dtype):
    """Stored KV-type array (uint16 bits for bf16, float32 for f32) -> float64."""
    if dtype == "bf16":
        return decode_bf16(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
