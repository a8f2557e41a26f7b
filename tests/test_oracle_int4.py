"""Pins for the oracle's 4-bit integer KV codec and its use in the cache and
attention oracles (CPU only).

The page (Worker-Side KV Init (zh), § KV Cache技术背景) fixes half a byte per
element; the format below it (zero point 8, nearest-even rounding, low nibble
first, per-tensor scale) is the reading stated in ``oracle/int4.py``.  The
expected values here are worked out by hand from that reading, or follow
from closed forms and brute force, never from the oracle itself.
"""

import numpy as np
import pytest

from oracle import attention, bf16, int4, paging, sizing


def test_encode_hand_examples():
    s = 0.5
    x = np.array([0.0, 0.25, 0.75, 1.25, -0.25, -0.75, 3.5, 3.75, 100.0, -100.0,
                  np.nan, -4.0, -4.25, np.inf, -np.inf, -0.0, 1.0, 3.2, -2.2], np.float32)
    # x / s:      0, 0.5, 1.5, 2.5, -0.5, -1.5, 7, 7.5, 200, -200, nan, -8, -8.5, inf, -inf, -0, 2, 6.4, -4.4
    want_k = [0, 0, 2, 2, 0, -2, 7, 7, 7, -8, 0, -8, -8, 7, -8, 0, 2, 6, -4]
    assert (int4.quantize(x, s).astype(int) - 8).tolist() == want_k


def test_pack_hand_example():
    codes = np.array([[1, 2, 15, 0, 8, 7]], np.uint8)
    assert int4.pack(codes).tolist() == [[0x21, 0x0F, 0x78]]
    np.testing.assert_array_equal(int4.unpack(np.array([[0x21, 0x0F, 0x78]], np.uint8)), codes)
    with pytest.raises(ValueError):
        int4.pack(np.zeros((2, 3), np.uint8))


def test_dequantize_hand_example():
    packed = np.array([0x0F, 0x80, 0x97], np.uint8)    # codes 15, 0, 0, 8, 7, 9
    np.testing.assert_array_equal(int4.dequantize(packed, 0.25),
                                  [1.75, -2.0, -2.0, 0.0, -0.25, 0.25])


@pytest.mark.parametrize("s", [0.5, 0.1, 0.0567, 3.0])
def test_levels_round_trip_exactly(s):
    """Every representable value k s (k in -8..7) encodes to k + 8 and
    decodes to k s (the scale as float32)."""
    k = np.arange(-8, 8)
    s32 = np.float64(np.float32(s))
    x = (k * s32).astype(np.float32)
    codes = int4.quantize(x, s)
    assert (codes.astype(int) - 8).tolist() == k.tolist()
    np.testing.assert_array_equal(int4.dequantize_codes(codes, s), k * s32)


def test_error_bound_monotone_and_saturation():
    rng = np.random.default_rng(5)
    s = 0.0371
    s32 = np.float64(np.float32(s))
    x = np.sort(rng.uniform(-8.5 * s, 7.5 * s, 20000).astype(np.float32))
    codes = int4.quantize(x, s)
    err = np.abs(int4.dequantize_codes(codes, s) - x.astype(np.float64))
    # half a step, plus the float32 rounding of x * (1 / s)
    assert err.max() <= 0.5 * s32 * (1 + 1e-6)
    assert (np.diff(codes.astype(int)) >= 0).all()
    big = np.array([7.6, 50, 1e30, -8.6, -50, -1e30], np.float32) * np.float32(s)
    assert (int4.quantize(big, s).astype(int) - 8).tolist() == [7, 7, 7, -8, -8, -8]


def test_bytes_per_token_is_a_quarter_of_fp16():
    """Half a byte per element against two for FP16 (the page's comparison),
    on the page's 80-layer / 8-head / 128-dim example."""
    b16 = sizing.kv_bytes_per_token(80, 8, 128, "bf16")
    assert sizing.kv_bytes_per_token(80, 8, 128, "int4") * 4 == b16 == 327680
    assert sizing.kv_bytes_per_token(80, 8, 128, "int4") * 2 == sizing.kv_bytes_per_token(80, 8, 128, "fp8")
    assert sizing.block_bytes(16, 8, 128, "int4") == 16 * 8 * 128   # K and V, half a byte each


def test_cache_write_packs_rows():
    """A bf16 row written to an int4 cache lands as hand-packed bytes."""
    bs, H, D = 4, 1, 4
    kp = np.zeros((3, bs, H, D // 2), np.uint8)
    vp = np.zeros_like(kp)
    key = bf16.from_f32(np.array([[[0.5, -0.5, 1.0, 3.6]]], np.float32))   # / 0.5: 1, -1, 2, 7.2
    val = bf16.from_f32(np.array([[[0.0, -4.0, 4.0, -0.25]]], np.float32))  # / 0.5: 0, -8, 8, -0.5
    k2, v2 = paging.cache_write(kp, vp, key, val, [6], "bf16", "int4", 0.5, 0.5)
    # codes k 9, 7, 10, 15 -> bytes 0x79, 0xFA;  v 8, 0, 15, 8 -> 0x08, 0x8F
    assert k2[1, 2, 0].tolist() == [0x79, 0xFA] and v2[1, 2, 0].tolist() == [0x08, 0x8F]
    assert k2.sum() == 0x79 + 0xFA and v2.sum() == 0x08 + 0x8F


def test_attention_over_int4_equals_attention_over_its_values():
    """Attention over an int4 cache built from integer codes equals attention
    over a float64 cache holding k * scale (the packing done here by hand)."""
    rng = np.random.default_rng(9)
    nb, bs, H, D, Hq = 6, 4, 2, 8, 4
    ks, vs = 0.125, 0.375
    kk = rng.integers(-8, 8, size=(nb, bs, H, D))
    vk = rng.integers(-8, 8, size=(nb, bs, H, D))

    def hand_pack(k):
        u = (k + 8).astype(np.int64)
        return (u[..., 0::2] + 16 * u[..., 1::2]).astype(np.uint8)

    q = bf16.from_f32(rng.standard_normal((3, Hq, D)).astype(np.float32))
    bt = np.array([[5, 1, 3], [0, 2, -1], [4, -1, -1]], np.int32)
    L = np.array([11, 6, 3], np.int32)
    a = attention.paged_decode(q, "bf16", hand_pack(kk), hand_pack(vk), "int4", bt, L, 0.4,
                               k_scale=ks, v_scale=vs)
    b = attention.paged_decode(q, "bf16", kk * ks, vk * vs, "f64", bt, L, 0.4)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)
