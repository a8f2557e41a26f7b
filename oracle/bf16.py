"""bfloat16 <-> float conversions written from the bit layout (oracle, test-only).

bfloat16 keeps the sign, the 8-bit exponent and the top 7 mantissa bits of an
IEEE-754 binary32 value.  Widening is therefore exact (append 16 zero bits);
narrowing rounds the 23-bit mantissa to 7 bits to nearest, ties to even.

The pages only say the cache holds FP16/BF16-class 2-byte elements (Worker-Side
KV Init (zh), § KV Cache技术背景: 2 bytes per element); the format itself is
the standard one.
"""

import numpy as np


def to_f64(bits):
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def from_f32(x):
    """float32 values -> uint16 bf16 bit patterns, round to nearest even.

    NaN stays NaN (quiet, sign kept); +-inf stay infinite; a finite value whose
    rounding carries past the largest exponent becomes infinite, as IEEE
    rounding prescribes.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(x)
    sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint32)
    rounded = np.where(nan, sign | np.uint32(0x7FC0), rounded)
    return rounded.astype(np.uint16)
