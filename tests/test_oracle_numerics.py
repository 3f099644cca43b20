"""Pins of the oracle's number formats against library conversions and
exhaustive enumeration (no GPU)."""
import numpy as np
import pytest
import torch

from oracle.numerics import (bf16_bits_to_f64, e4m3_decode, e4m3_encode,
                             e4m3_quantize, f64_to_bf16_bits, round_bf16)


def _torch_bf16(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_rne_matches_torch_sweep():
    g = np.random.default_rng(0)
    mant = g.uniform(1.0, 2.0, 200000)
    expo = g.integers(-140, 127, 200000)
    x = (np.ldexp(mant, expo) * np.where(g.random(200000) < 0.5, -1, 1)).astype(np.float32)
    np.testing.assert_array_equal(round_bf16(x.astype(np.float64)), _torch_bf16(x))


def test_bf16_ties_to_even_and_edges():
    # exact midpoints between consecutive bf16 values: lower mantissa even -> round down
    base = np.arange(0x3F80, 0x3FFF, dtype=np.uint16)          # [1, 2)
    lo = bf16_bits_to_f64(base)
    hi = bf16_bits_to_f64(base + 1)
    mid = (lo + hi) / 2
    r = round_bf16(mid)
    even = np.where(base % 2 == 0, lo, hi)
    np.testing.assert_array_equal(r, even)
    np.testing.assert_array_equal(r, _torch_bf16(mid.astype(np.float32)))
    # overflow to inf, subnormals, signed zero, nan
    big = np.float64(np.finfo(np.float32).max)
    assert round_bf16(big) == np.inf and round_bf16(-big) == -np.inf
    tiny = np.float32(3e-40)
    assert round_bf16(np.float64(tiny)) == _torch_bf16(np.array([tiny]))[0]
    assert np.isnan(round_bf16(np.nan))
    assert np.signbit(round_bf16(-0.0))


def test_bf16_bits_roundtrip_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(vals), np.isnan(ref))
    fin = np.isfinite(vals)
    np.testing.assert_array_equal(vals[fin], ref[fin])
    np.testing.assert_array_equal(f64_to_bf16_bits(vals[fin]), bits[fin])


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(mine[ok], ref[ok])
    assert np.nanmax(mine) == 448.0 and np.nanmin(mine) == -448.0
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    assert mine[0x01] == 2.0 ** -9                # smallest subnormal


def test_e4m3_encode_roundtrip_and_midpoints():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(codes)), codes)
    # midpoints of consecutive positive finite codes round to the even code
    pos = np.arange(0x00, 0x7E, dtype=np.uint8)
    mid = (e4m3_decode(pos) + e4m3_decode(pos + 1)) / 2
    want = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    np.testing.assert_array_equal(e4m3_encode(mid), want)
    np.testing.assert_array_equal(e4m3_encode(-mid), want | 0x80)


def test_e4m3_saturates():
    for v, c in [(448.0, 0x7E), (449.0, 0x7E), (464.0, 0x7E), (1e9, 0x7E),
                 (-1e9, 0xFE), (np.inf, 0x7E)]:
        assert e4m3_encode(v) == c, v


def test_e4m3_encode_matches_torch_in_range():
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(100000) * 50, g.standard_normal(20000) * 0.01])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_encode(x.astype(np.float64)), ref)


def test_e4m3_quantize_divides_in_fp32():
    g = np.random.default_rng(2)
    x = g.standard_normal(10000)
    scale = 0.0123
    want = torch.from_numpy((x.astype(np.float32) / np.float32(scale)).clip(-448, 448)) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_quantize(x, scale), want)
