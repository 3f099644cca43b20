"""Number formats used at the layer's rounding points, written from their
definitions (test infrastructure only; see oracle/__init__.py).

* bf16: 1 sign, 8 exponent, 7 stored mantissa bits (8 significant bits), same
  exponent range as IEEE binary32; round-to-nearest-even, overflow to inf.
* fp8 e4m3 "FN" (OCP 8-bit floating point spec, the format gfx950 uses): 1 sign,
  4 exponent (bias 7), 3 mantissa bits; no infinities, S.1111.111 is NaN, so the
  largest finite magnitude is 1.75 * 2^8 = 448; exponent field 0 encodes
  subnormals M/8 * 2^-6. Encoding here rounds to nearest even and saturates to
  +-448 (the KV-cache write of Beam's fp8 cache, "Attention" section of the
  Reflection Beam pages: the cache may be stored in FP8).

Everything is computed in float64; a rounding function returns float64 values
that are exactly representable in the target format.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even)."""
    x = np.asarray(x, dtype=F64)
    a = np.abs(x)
    _, e = np.frexp(a)                      # 2**(e-1) <= a < 2**e
    ulp_exp = np.maximum(e - 8, -133)       # 8 significant bits; subnormal ulp 2**-133
    r = np.ldexp(np.rint(np.ldexp(x, -ulp_exp)), ulp_exp)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode raw bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(F64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Encode float64 values that are already bf16-exact to their bit patterns."""
    r = round_bf16(x).astype(np.float32)    # exact: bf16 values are fp32 values
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=F64).astype(np.float32).astype(F64)


E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of every e4m3fn code (float64); the two NaN codes decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    mag = np.where(E == 0, M / 8.0 * 2.0 ** -6, (1.0 + M / 8.0) * np.exp2(E - 7.0))
    mag = np.where((E == 15) & (M == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """Round to the nearest e4m3fn value (ties to even), saturating at +-448."""
    x = np.asarray(x, dtype=F64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, e = np.frexp(a)                      # 2**(e-1) <= a < 2**e
    ulp_exp = np.maximum(e - 4, -9)         # 4 significant bits; subnormal ulp 2**-9
    q = np.minimum(np.ldexp(np.rint(np.ldexp(a, -ulp_exp)), ulp_exp), E4M3_MAX)
    # value -> code
    sub = q < 2.0 ** -6
    _, eq = np.frexp(np.where(sub, 1.0, q))
    E = np.where(sub, 0, eq - 1 + 7)
    M = np.where(sub, np.rint(q / 2.0 ** -9), np.rint((np.ldexp(q, -(eq - 1)) - 1.0) * 8.0))
    code = (E.astype(np.int64) << 3) | M.astype(np.int64)
    code = np.where(neg, code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def e4m3_quantize(x, scale: float) -> np.ndarray:
    """Cache code of x under a per-tensor scale. The division and the rounding
    decision are taken in binary32, the precision the cache writer works in."""
    x32 = np.asarray(x, dtype=F64).astype(np.float32)
    return e4m3_encode((x32 / np.float32(scale)).astype(F64))
