"""Pins of the oracle's storage codecs against torch's library casts and the
format definitions (exhaustive over every code)."""
import numpy as np
import pytest
import torch

from oracle import codecs


def test_bf16_decode_all_codes_match_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours), bits >= 0x8000)   # NaNs included
    # Signed zeros and infinities sit where the definition puts them.
    assert ours[0x0000] == 0.0 and np.signbit(ours[0x8000])
    assert ours[0x7F80] == np.inf and ours[0xFF80] == -np.inf
    assert ours[0x3F80] == 1.0 and ours[0x0001] == 2.0 ** -133


def test_f32_decode_is_exact():
    x = np.array([0.0, -0.0, 1.5, -3.25e-38, 1e-45, 3.4e38], dtype=np.float32)
    assert np.array_equal(codecs.f32_to_f64(x.view(np.uint32)), x.astype(np.float64))


def test_e4m3fn_decode_all_codes_match_torch():
    bits = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3fn_to_f64(bits)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # Definition landmarks: only S.1111.111 is NaN, 448 is the largest
    # magnitude, 2^-9 the smallest subnormal, 2^-6 the smallest normal.
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(np.signbit(ours), bits >= 0x80)     # NaNs included
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert np.all(np.diff(ours[:0x7F]) > 0)  # monotone over the positive codes


def test_e4m3fn_encode_round_trips_every_finite_code():
    bits = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = codecs.e4m3fn_to_f64(bits).astype(np.float32)
    assert np.array_equal(codecs.f32_to_e4m3fn(vals), bits)


def test_e4m3fn_encode_matches_torch_cast_after_clamp():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 50,
        rng.standard_normal(20000).astype(np.float32) * 2.0 ** -7,  # subnormal range
        rng.uniform(-600, 600, 20000).astype(np.float32),
        np.array([0.0, -0.0, 448.0, -448.0, 449.0, 464.0, 1e30, -1e30], dtype=np.float32),
    ])
    ours = codecs.f32_to_e4m3fn(x)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3fn_encode_ties_go_to_even_code():
    pos = codecs.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)  # exact in f32
    codes = codecs.f32_to_e4m3fn(mids).astype(int)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes, expect)
    # Just off the midpoint the nearer code wins regardless of parity.
    up = codecs.f32_to_e4m3fn(np.nextafter(mids, np.float32(1e9)))
    assert np.array_equal(up.astype(int), lo + 1)


def test_e4m3fn_encode_specials():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf, 1e-30, -1e-30], dtype=np.float32)
    x[1] = -np.abs(x[1])
    out = codecs.f32_to_e4m3fn(x)
    assert out[0] == 0x7F and out[1] == 0xFF
    assert out[2] == 0x7E and out[3] == 0xFE      # saturating
    assert out[4] == 0x00 and out[5] == 0x80      # underflow keeps the sign


def test_quantize_divides_in_float32_then_encodes():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(50000).astype(np.float32) * 4
    scale = np.float32(np.abs(x).max() / np.float32(448.0))
    ours = codecs.quantize_e4m3fn(x, scale)
    q = torch.from_numpy(x) / torch.tensor(scale, dtype=torch.float32)
    ref = q.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # Dequantised error stays within half an fp8 step (relative 2^-4) plus the subnormal floor.
    back = codecs.e4m3fn_to_f64(ours) * float(scale)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -4 + float(scale) * 2.0 ** -10)


def test_decode_dispatch_applies_fp8_scale_only():
    assert codecs.decode(np.array([0x38], np.uint8), "fp8", 0.5)[0] == 0.5
    assert codecs.decode(np.array([0x3F80], np.uint16), "bf16", 0.5)[0] == 1.0
    with pytest.raises(ValueError):
        codecs.decode(np.array([0], np.uint8), "int8")


def test_nan_sign_survives_decode_and_quantise():
    # A negative NaN stays negative through decode and the fp8 quantiser.
    for bits, dt in ((np.array([0xFFC0], np.uint16), "bf16"), (np.array([0xFF], np.uint8), "fp8")):
        x = codecs.decode(bits, dt).astype(np.float32)
        assert np.isnan(x[0]) and np.signbit(x[0])
        assert codecs.quantize_e4m3fn(x, 0.5)[0] == 0xFF
