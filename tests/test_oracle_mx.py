"""Pins of the MXFP8 block codec (oracle/mx.py) against its definition: closed
forms of the shared exponent, exact round trips of representable blocks,
brute-force nearest-value search, the error bound, saturation and zero blocks."""
import numpy as np

from oracle import mx
from oracle.numerics import e4m3_decode

ALL = np.arange(256, dtype=np.uint8)
FINITE = ALL[~np.isnan(e4m3_decode(ALL))]          # every finite e4m3 code


def test_shared_exponent_closed_forms():
    # s = floor(log2(amax)) - 8
    cases = {1.0: -8, 448.0: 0, 511.0: 0, 512.0: 1, 0.02: -14, 3e-5: -24, 2.0 ** -120: -127}
    for amax, s in cases.items():
        block = np.zeros(32)
        block[7] = -amax
        block[3] = amax / 3
        assert mx.shared_exponents(block)[0] == s, (amax, s)


def test_zero_block():
    codes, scales = mx.mxfp8_quantize(np.zeros((2, 64)))
    assert np.all(codes == 0) and np.all(scales == 0)      # s = -127
    assert np.all(mx.mxfp8_dequantize(codes, scales) == 0)


def test_representable_blocks_round_trip_exactly():
    g = np.random.default_rng(0)
    for s in (-20, -10, 0, 5):
        c = g.choice(FINITE, size=(4, 64))
        c[:, 0] = 0x7E                                     # 448: the block max sets X
        c[:, 32] = 0xFE                                    # -448
        w = np.ldexp(e4m3_decode(c), s)
        codes, scales = mx.mxfp8_quantize(w)
        assert np.all(scales.astype(int) - 127 == s)
        np.testing.assert_array_equal(mx.mxfp8_dequantize(codes, scales), w)


def test_nearest_value_by_enumeration():
    """Every code is the nearest finite e4m3 value of w / X (ties to the even
    code, i.e. the one with a zero last mantissa bit), found by brute force."""
    g = np.random.default_rng(1)
    w = g.standard_normal((8, 96)) * 0.02
    w[0, :32] = np.linspace(-1, 1, 32) * 3e-4               # a block with subnormal codes
    codes, scales = mx.mxfp8_quantize(w)
    vals = e4m3_decode(FINITE)
    for r in range(w.shape[0]):
        for b in range(w.shape[1] // 32):
            X = 2.0 ** (int(scales[r, b]) - 127)
            for k in range(32):
                x = w[r, 32 * b + k] / X
                d = np.abs(vals - min(max(x, -448.0), 448.0))
                best = FINITE[d == d.min()]
                if len(best) > 1:                           # a tie: the even mantissa
                    best = best[(best & 1) == 0]
                assert codes[r, 32 * b + k] in best, (r, b, k, x)


def test_error_bound_and_saturation():
    g = np.random.default_rng(2)
    w = g.standard_normal((16, 256)) * 0.02
    codes, scales = mx.mxfp8_quantize(w)
    d = mx.mxfp8_dequantize(codes, scales)
    X = np.repeat(2.0 ** (scales.astype(int) - 127), 32, axis=1)
    x = np.abs(w) / X
    err = np.abs(d - w) / X
    normal = (x >= 2.0 ** -6) & (x <= 448)
    assert np.all(err[normal] <= 2.0 ** -4 * x[normal] + 1e-12)   # half an ulp of 3 bits
    assert np.all(err[x < 2.0 ** -6] <= 2.0 ** -10 + 1e-15)      # half the subnormal step
    # amax / X is in [256, 512): values above 448 clamp to the largest code
    block = np.full(32, 1.0)
    block[0] = 500.0 / 256.0                                      # X = 2^-8, 500 -> 448
    c, s = mx.mxfp8_quantize(block)
    assert int(s[0]) - 127 == -8 and c[0] == 0x7E
    assert mx.mxfp8_dequantize(c, s)[0] == 448.0 / 256.0
