"""OCP 8-bit floating point E4M3 ("FN" variant) codec (oracle, test-only).

The pages say only that an FP8 KV cache stores one byte per element instead
of two and so halves KV memory (Worker-Side KV Init (zh), § KV Cache技术背景).
Which FP8 is meant is left open; the reading taken here is the OCP E4M3FN
format that gfx950 hardware implements:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 is subnormal: value = mantissa/8 * 2**-6;
* no infinities; the only NaN patterns are S.1111.111 (0x7F, 0xFF);
* largest finite magnitude 1.75 * 2**8 = 448, smallest subnormal 2**-9.

Quantisation of a cache element x with per-tensor scale s:
    code = encode(float32(x) * inv_s),  inv_s = float32(1 / float32(s))
with round-to-nearest, ties to the even mantissa, saturation of every
finite magnitude above 448 to +-448 (infinite inputs too), NaN -> NaN.
Dequantisation: x_hat = decode(code) * s.

``encode`` searches the 256-entry table for the nearest value; it does not use
bit tricks, so it is independent of any shift-and-round implementation.
"""

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def decode_table():
    """float64[256]: value of every code, built from the bit definition."""
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = (code >> 7) & 1
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            v = np.nan
        elif e == 0:
            v = (m / 8.0) * 2.0 ** (-6)
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        tab[code] = -v if s else v
    return tab


_TABLE = decode_table()
# Non-negative finite codes 0x00..0x7E in increasing value order.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = _TABLE[:0x7F]


def decode(codes):
    """uint8 codes -> float64 values (exact)."""
    return _TABLE[np.asarray(codes).astype(np.int64)]


def encode(x):
    """float32 values -> uint8 codes (nearest, ties to even, saturating).

    The argument is taken as float32 (the type in which the product of the
    element and the inverse scale is formed) and compared exactly in float64.
    """
    x32 = np.asarray(x, dtype=np.float32)
    flat = x32.reshape(-1).astype(np.float64)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, v in enumerate(flat):
        if np.isnan(v):
            out[i] = NAN_CODE | (0x80 if np.signbit(v) else 0)
            continue
        sign = 0x80 if np.signbit(v) else 0
        a = abs(v)
        if a >= MAX_FINITE:
            out[i] = sign | 0x7E
            continue
        # nearest representable magnitude; on a tie take the even mantissa
        d = np.abs(_POS_VALUES - a)
        best = d.min()
        cand = _POS_CODES[d == best]
        if len(cand) > 1:
            cand = cand[(cand & 1) == 0]
        out[i] = sign | int(cand[0])
    return out.reshape(x32.shape)


def encode_fast(x):
    """Vectorised equivalent of :func:`encode` for large arrays.

    Same rule (nearest table value, ties to even, saturate, NaN kept) done by
    binary search over the sorted non-negative table; tests check it equal to
    :func:`encode` on every input they give the scalar version.
    """
    x32 = np.asarray(x, dtype=np.float32)
    v = x32.astype(np.float64)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    a = np.abs(v)
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    dlo = np.abs(a - _POS_VALUES[lo])
    dhi = np.abs(_POS_VALUES[hi] - a)
    pick_lo = (dlo < dhi) | ((dlo == dhi) & ((lo & 1) == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = np.where(a >= MAX_FINITE, np.uint8(0x7E), code)
    code = (code | sign).astype(np.uint8)
    code = np.where(np.isnan(v), (NAN_CODE | sign).astype(np.uint8), code)
    return code.astype(np.uint8)


def inv_scale(scale):
    """The float32 inverse scale both sides multiply by: float32(1/float32(s))."""
    return np.float32(1.0) / np.float32(scale)


def quantize(x, scale):
    """float32 elements -> e4m3 codes with a per-tensor scale."""
    with np.errstate(over="ignore", invalid="ignore"):   # inf/NaN inputs stay inf/NaN
        prod = (np.asarray(x, dtype=np.float32) * inv_scale(scale)).astype(np.float32)
    return encode_fast(prod)


def dequantize(codes, scale):
    """e4m3 codes -> float64 values times the per-tensor scale."""
    return decode(codes) * np.float64(np.float32(scale))
