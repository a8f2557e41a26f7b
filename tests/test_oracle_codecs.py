"""Pins for the oracle's bf16 and OCP E4M3 codecs (CPU only)."""

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3


def test_e4m3_decode_table_landmarks():
    t = e4m3.decode_table()
    assert t[0x00] == 0.0 and np.signbit(t[0x80])      # +0, -0
    assert t[0x38] == 1.0                                # exponent 7 = bias
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0        # largest finite
    assert t[0x08] == 2.0 ** -6                          # smallest normal
    assert t[0x01] == 2.0 ** -9                          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9                      # largest subnormal
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])       # the only NaNs
    assert np.isfinite(np.delete(t, [0x7F, 0xFF])).all()
    pos = t[:0x7F]
    assert (np.diff(pos) > 0).all()                      # monotone codes


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.decode(np.arange(256))
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert (both_nan | (ref == ours)).all()
    assert (np.signbit(ref) == np.signbit(ours))[~both_nan].all()


def test_e4m3_encode_inverts_decode():
    t = e4m3.decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])])
    assert (e4m3.encode(t[codes].astype(np.float32)) == codes).all()
    assert (e4m3.encode_fast(t[codes].astype(np.float32)) == codes).all()


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),            # halfway 1.0 / 1.125 -> even mantissa (1.0)
    (1.1875, 0x3A),            # halfway 1.125 / 1.25 -> even (1.25)
    (17.0, 0x58),              # halfway 16 / 18 -> 16
    (19.0, 0x5A),              # halfway 18 / 20 -> 20
    (2.0 ** -10, 0x00),        # halfway 0 / 2^-9 -> 0
    (3 * 2.0 ** -10, 0x02),    # halfway 2^-9 / 2^-8 -> 2^-8
    (464.0, 0x7E),             # past the largest finite: saturate
    (1e30, 0x7E),
    (float("inf"), 0x7E),
    (-1e30, 0xFE),
    (-0.0, 0x80),
])
def test_e4m3_encode_rounding_and_saturation(x, code):
    assert int(e4m3.encode(np.float32(x))) == code
    assert int(e4m3.encode_fast(np.float32(x))) == code


def test_e4m3_encode_nan():
    assert int(e4m3.encode(np.float32(np.nan))) & 0x7F == 0x7F
    assert int(e4m3.encode_fast(np.float32(-np.nan))) == 0xFF


def test_e4m3_encode_matches_torch_on_all_bf16_inputs_within_range():
    bits = np.arange(65536, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x)]
    clamped = np.clip(x, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = e4m3.encode_fast(clamped)
    assert (ref == ours).all()
    # and saturation beyond the clamp: our encoder saturates without help
    assert (e4m3.encode_fast(x) == ref).all()


def test_e4m3_scalar_and_vector_encoders_agree():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.uniform(-4, 3, 3000),
                        [0.0, -0.0, 448.0, 449.0, 2.0 ** -9, 2.0 ** -10]]).astype(np.float32)
    assert (e4m3.encode(x) == e4m3.encode_fast(x)).all()


def test_e4m3_quantize_uses_float32_inverse_scale():
    s = np.float32(0.37)
    inv = e4m3.inv_scale(s)
    assert inv.dtype == np.float32 and inv == np.float32(1.0) / s
    x = np.array([1.0, -2.5, 100.0], dtype=np.float32)
    assert (e4m3.quantize(x, s) == e4m3.encode_fast((x * inv).astype(np.float32))).all()
    # dequantised error bounded by half an e4m3 ulp (3 mantissa bits) times scale
    rng = np.random.default_rng(4)
    y = rng.standard_normal(10000).astype(np.float32)
    sc = np.float32(np.abs(y).max() / 448.0)
    back = e4m3.dequantize(e4m3.quantize(y, sc), sc)
    rel = np.abs(back - y) / np.maximum(np.abs(y), 2.0 ** -6 * sc)
    assert rel.max() <= 2.0 ** -4 + 1e-6


def test_bf16_widen_and_round_to_nearest_even():
    assert bf16.to_f64(np.uint16(0x3F80)) == 1.0
    assert bf16.to_f64(np.uint16(0xC000)) == -2.0
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7 -> even (1.0)
    assert bf16.from_f32(np.float32(1 + 2.0 ** -8)) == 0x3F80
    assert bf16.from_f32(np.float32(1 + 3 * 2.0 ** -8)) == 0x3F82
    assert bf16.from_f32(np.float32(np.inf)) == 0x7F80
    assert (bf16.from_f32(np.float32(np.nan)) & 0x7FC0) == 0x7FC0


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-30, 30, 200000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (bf16.from_f32(x) == ref).all()
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert (bf16.to_f64(ref) == back).all()
