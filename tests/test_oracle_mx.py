"""Pins of the MXFP8 and MXFP4 block codecs (oracle/mx.py) against their
definition: closed forms of the shared exponent, the E2M1 value set, exact
round trips of representable blocks, nearest-value search by brute force and by
midpoints, the error bound, saturation, zero blocks and the nibble order."""
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


# ------------------------------------------------------------------ MXFP4 (E2M1)
def test_e2m1_value_set():
    # OCP MX: E2M1 has max normal 6.0, min normal 1.0, min subnormal 0.5
    v = mx.e2m1_decode(np.arange(16))
    assert list(v[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(v[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert np.signbit(v[8])
    for c in range(16):                                         # exact round trip
        assert mx.e2m1_encode(v[c]) == c


def test_e2m1_nearest_by_midpoints():
    """Independent of the encoder's search: a magnitude's code is the number of
    midpoints between consecutive values that lie below it; on a midpoint the
    even code (zero mantissa bit) wins; above 6 the code saturates."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    g = np.random.default_rng(3)
    a = np.concatenate([g.uniform(0, 9, 4000), mids, [0.0, 6.0, 7.999, 1e9]])
    for x in a:
        if x in mids:                                            # between codes i and i+1
            i = mids.index(x)
            c = i if i % 2 == 0 else i + 1
        else:
            c = sum(x > m for m in mids)
        assert mx.e2m1_encode(x) == c, x
        assert mx.e2m1_encode(-x) == c | 8, x


def test_mxfp4_shared_exponent_and_zero_block():
    # s = floor(log2(amax)) - 2
    for amax, s in {1.0: -2, 6.0: 0, 7.9: 0, 8.0: 1, 0.02: -8, 2.0 ** -126: -127}.items():
        block = np.zeros(32)
        block[11] = -amax
        assert mx.shared_exponents(block, mx.E2M1_EMAX)[0] == s, (amax, s)
    p, sc = mx.mxfp4_quantize(np.zeros((3, 64)))
    assert p.shape == (3, 32) and sc.shape == (3, 2)
    assert np.all(p == 0) and np.all(sc == 0)
    assert np.all(mx.mxfp4_dequantize(p, sc) == 0)


def test_mxfp4_nibble_order_and_round_trip():
    g = np.random.default_rng(4)
    for s in (-12, -3, 0, 7):
        c = g.integers(0, 16, size=(5, 96))
        c[:, 0] = 7                                              # 6: the block max sets X
        c[:, 32] = 15
        c[:, 64] = 7
        w = np.ldexp(mx.e2m1_decode(c), s)
        p, sc = mx.mxfp4_quantize(w)
        assert np.all(sc.astype(int) - 127 == s)
        assert np.all(p == ((c[:, 0::2] & 15) | ((c[:, 1::2] & 15) << 4)))
        np.testing.assert_array_equal(mx.mxfp4_dequantize(p, sc), w)
    w = np.zeros(32)
    w[0], w[1] = 6.0, -0.5                                       # X = 1
    p, _ = mx.mxfp4_quantize(w)
    assert p[0] == 0x7 | (0x9 << 4)


def test_mxfp4_error_bound_and_saturation():
    g = np.random.default_rng(5)
    w = g.standard_normal((16, 256)) * 0.02
    p, sc = mx.mxfp4_quantize(w)
    d = mx.mxfp4_dequantize(p, sc)
    X = np.repeat(2.0 ** (sc.astype(int) - 127), 32, axis=1)
    x = np.abs(w) / X
    err = np.abs(d - w) / X
    assert np.all(x < 8)
    half_step = np.where(x < 2, 0.25, np.where(x < 4, 0.5, 1.0))
    ok = x <= 6
    assert np.all(err[ok] <= half_step[ok])
    assert np.all(err[~ok] == x[~ok] - 6)                         # saturated to 6
    block = np.full(32, 0.5)
    block[0] = 7.5                                               # X = 1, 7.5 -> 6
    p, s = mx.mxfp4_quantize(block)
    assert int(s[0]) == 127 and (p[0] & 15) == 7
    assert mx.mxfp4_dequantize(p, s)[0] == 6.0


# ---- block-scaled operands on both sides (scaled matrix-core experts) --------
def _tiny_moe_case(seed=5):
    import synth
    from oracle import layer as L
    dims = synth.with_dims(synth.config(0), F=64, E=4, topk=2, n_group=1, topk_group=1).dims
    g = np.random.default_rng(seed)
    T = 5
    x = L.bf(g.standard_normal((T, dims.D)))
    idx = np.stack([g.choice(dims.E, dims.topk, replace=False) for _ in range(T)])
    w = g.uniform(0.1, 0.9, (T, dims.topk)).astype(np.float32)
    ex = {e: (L.bf(g.standard_normal((2 * dims.F, dims.D)) * 0.05),
              L.bf(g.standard_normal((dims.D, dims.F)) * 0.05)) for e in range(dims.E)}
    return dims, x, idx, w, ex


def test_mxfp8_round_is_a_projection():
    """Quantising twice gives the first result; representable blocks are
    fixed points; the error stays within half an e4m3 step of the block."""
    g = np.random.default_rng(1)
    a = g.standard_normal((7, 96)) * np.exp(g.uniform(-8, 8, (7, 1)))
    r = mx.mxfp8_round(a)
    assert np.array_equal(mx.mxfp8_round(r), r)
    s = mx.shared_exponents(a)[..., None]
    X = np.ldexp(1.0, s)                          # block scale
    half = np.ldexp(1.0, s + 8 - 3 - 1)          # half the e4m3 spacing of the top binade
    a3, r3 = a.reshape(7, 3, 32), r.reshape(7, 3, 32)
    inside = np.abs(a3) <= 448 * X
    assert np.all(np.abs(r3 - a3)[inside] <= (half * np.ones_like(a3))[inside] * 1.0000001)
    assert np.array_equal(r3[~inside], (np.sign(a3) * 448 * X)[~inside])   # saturation


def test_moe_mx_scaled_reduces_to_the_bf16_moe():
    """With an identity quantiser the scaled MoE is the pinned bf16 MoE on the
    same weights, bit for bit: the two differ only in the quantiser calls."""
    from oracle import layer as L
    dims, x, idx, w, ex = _tiny_moe_case()
    ident = mx.moe_mx_scaled(dims, x, idx, w, lambda e: ex[e], q=lambda a: np.asarray(a))
    assert np.array_equal(ident, L.moe(dims, x, idx, w, lambda e: ex[e]))


def test_moe_mx_scaled_quantises_both_product_inputs():
    """The quantiser sees the token rows (x, [T][D]) once and each expert's
    activation rows ([rows][F]) before its down product, and nothing else;
    quantising x beforehand changes nothing (the first call is a projection)."""
    dims, x, idx, w, ex = _tiny_moe_case(7)
    seen = []

    def spy(a):
        seen.append(np.asarray(a).shape)
        return mx.mxfp8_round(a)
    y = mx.moe_mx_scaled(dims, x, idx, w, lambda e: ex[e], q=spy)
    n_e = [int(np.sum(idx == e)) for e in np.unique(idx)]
    assert seen == [x.shape] + [(n, dims.F) for n in n_e]
    assert np.array_equal(mx.moe_mx_scaled(dims, mx.mxfp8_round(x), idx, w, lambda e: ex[e]), y)
    # and it matters: the scaled result differs from the unscaled one
    from oracle import layer as L
    assert not np.array_equal(y, L.moe(dims, x, idx, w, lambda e: ex[e]))
