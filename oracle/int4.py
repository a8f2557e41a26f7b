"""4-bit integer KV-cache codec (oracle, test-only).

Page: Worker-Side KV Init (zh), § KV Cache技术背景 -- an INT4 cache stores
half a byte per element (a quarter of FP16) and may need calibration data to
keep accuracy; § 第一步：物理分配 -- the cache is a plain byte array viewed in
whatever element type the layer uses, so an INT4 layer packs two elements in
each byte.

The pages fix nothing else.  Readings taken here:

* Element value = (u - 8) * s: u is the unsigned 4-bit code 0..15 (zero
  point 8, so values -8 s .. 7 s) and s a per-tensor scale that is chosen
  offline -- the calibration the page speaks of; the synthetic workloads
  draw codes directly and take s = sigma / 2 (sigma the data's standard
  deviation, 1 / sqrt(128) for the Llama-shaped workloads).  Nothing about
  s is computed at write time.
* Quantisation: y = float32(x) * inv_s with inv_s = float32(1 / float32(s))
  (the float32 product, as for the FP8 cache); k = the integer nearest to y,
  ties to the even integer, limited to [-8, 7]; u = k + 8.  A NaN element
  stores u = 8 (value 0): the format has no NaN.
* Packing: element 2j of a row sits in the low nibble of byte j, element
  2j + 1 in the high nibble.  A row of D elements takes D / 2 bytes.

``encode`` picks the nearest of the sixteen representable integers by
search, not by a rounding instruction, so it is independent of any
shift-and-round implementation.
"""

import numpy as np

ZERO_POINT = 8
_LEVELS = np.arange(-8, 8, dtype=np.float64)      # the representable integers


def inv_scale(scale):
    """The float32 inverse scale the quantiser multiplies by."""
    return np.float32(1.0) / np.float32(scale)


def encode(y):
    """float32 values (already divided by the scale) -> codes u in 0..15.

    Nearest representable integer, ties to the even one; values beyond the
    range go to the nearest end; NaN -> 8.
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    flat = y.reshape(-1)
    nan = np.isnan(flat)
    # beyond the range the nearest level is the end one; clipping to one step
    # past each end keeps it so and makes infinities finite
    v = np.clip(np.where(nan, 0.0, flat), -9.0, 8.0)
    d = np.abs(_LEVELS[None, :] - v[:, None])          # distance to every level
    near = d == d.min(axis=1, keepdims=True)            # one level, or two at a tie
    even = near & ((_LEVELS.astype(np.int64) % 2) == 0)[None, :]
    pick = np.where(even.any(axis=1), even.argmax(axis=1), near.argmax(axis=1))
    k = _LEVELS[pick].astype(np.int64)
    out = np.where(nan, ZERO_POINT, k + ZERO_POINT).astype(np.uint8)
    return out.reshape(y.shape)


def quantize(x, scale):
    """float32 elements -> codes u (uint8, one per element) with a per-tensor scale."""
    with np.errstate(over="ignore", invalid="ignore"):
        prod = (np.asarray(x, dtype=np.float32) * inv_scale(scale)).astype(np.float32)
    return encode(prod)


def dequantize_codes(codes, scale):
    """Codes u -> float64 values (u - 8) * s."""
    return (np.asarray(codes).astype(np.float64) - ZERO_POINT) * np.float64(np.float32(scale))


def pack(codes):
    """[..., D] codes (D even) -> [..., D / 2] bytes, low nibble first."""
    c = np.asarray(codes).astype(np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("an INT4 row needs an even number of elements")
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack(packed):
    """[..., D / 2] bytes -> [..., D] codes."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def quantize_packed(x, scale):
    """float32 rows [..., D] -> packed bytes [..., D / 2]."""
    return pack(quantize(x, scale))


def dequantize(packed, scale):
    """Packed bytes [..., D / 2] -> float64 values [..., D]."""
    return dequantize_codes(unpack(packed), scale)
