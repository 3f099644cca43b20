"""MXFP8 and MXFP4 block quantisation of expert weights, written from the
OCP Microscaling (MX) format definition (test infrastructure only; see
oracle/__init__.py).

The pages run the routed experts in a 4-bit block format ("Reflection Beam
1.0 on vLLM", MoE section: the experts' d_ff is given in NVFP4; the library
MoE path of the optimisation section quantises for it). The MI355X-native
counterpart used here keeps 8-bit elements:

* a block is 32 consecutive weights along the reduction (K) axis of one row;
* every block shares one scale X = 2^s, stored as an E8M0 byte s + 127
  (s in [-127, 127]);
* s = floor(log2(amax)) - 8, amax the block's largest magnitude and 8 the
  exponent of the largest normal E4M3 value (448 = 1.75 * 2^8), so amax / X
  lies in [256, 512); a block of zeros takes s = -127;
* each element is the E4M3 code of w / X, rounded to nearest even and
  saturated at +-448 (magnitudes in (448, 512) clamp);
* the weight a kernel uses is decode(code) * X.

MXFP4 follows the same scheme with E2M1 elements (1 sign, 2 exponent bits with
bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6): s =
floor(log2(amax)) - 2 (2 = the exponent of the largest E2M1 value), so amax / X
lies in [4, 8) and magnitudes above 6 clamp; two codes share a byte, element 2i
in the low nibble and 2i + 1 in the high one.

w / X is exact (X is a power of two inside the float64 range), so the only
rounding is the E4M3 encoding, the same in any precision that holds w.
"""
from __future__ import annotations

import numpy as np

from .numerics import e4m3_decode, e4m3_encode

F64 = np.float64
BLOCK = 32
E4M3_EMAX = 8
E2M1_EMAX = 2


def shared_exponents(w, emax: int = E4M3_EMAX) -> np.ndarray:
    """Scale exponent s of every 32-element block along the last axis, for an
    element format whose largest value has exponent emax."""
    w = np.asarray(w, dtype=F64)
    assert w.shape[-1] % BLOCK == 0, "K must be a multiple of 32"
    amax = np.abs(w.reshape(*w.shape[:-1], w.shape[-1] // BLOCK, BLOCK)).max(axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))   # 2**(e-1) <= amax < 2**e
    s = (e - 1) - emax
    s = np.where(amax > 0, s, -127)
    return np.clip(s, -127, 127).astype(np.int64)


def mxfp8_quantize(w):
    """(codes uint8 [..., K], scales uint8 [..., K/32]) of weights w [..., K]."""
    w = np.asarray(w, dtype=F64)
    s = shared_exponents(w)
    x = np.ldexp(w.reshape(*w.shape[:-1], -1, BLOCK), -s[..., None])
    codes = e4m3_encode(x).reshape(w.shape)
    return codes.astype(np.uint8), (s + 127).astype(np.uint8)


def mxfp8_dequantize(codes, scales) -> np.ndarray:
    """The weights a kernel multiplies with: decode(code) * 2^(scale - 127)."""
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.int64) - 127
    v = e4m3_decode(c).reshape(*c.shape[:-1], -1, BLOCK)
    return np.ldexp(v, s[..., None]).reshape(c.shape)


# ---------------------------------------------------------------------------
# E2M1 elements (MXFP4)
# ---------------------------------------------------------------------------

def e2m1_magnitudes() -> np.ndarray:
    """Value of the magnitude codes 0..7 from the field layout: exponent field
    e (bias 1) and mantissa bit m give m / 2 for e = 0 (subnormal) and
    (1 + m / 2) * 2^(e - 1) otherwise."""
    v = []
    for code in range(8):
        e, m = code >> 1, code & 1
        v.append(m / 2.0 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return np.array(v, F64)


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    v = e2m1_magnitudes()[c & 7]
    return np.where(c & 8, -v, v)


def e2m1_encode(x) -> np.ndarray:
    """Nearest E2M1 value, ties to the even code, magnitudes above 6 saturate."""
    x = np.asarray(x, dtype=F64)
    a = np.minimum(np.abs(x), 6.0)
    mags = e2m1_magnitudes()
    d = np.abs(a[..., None] - mags)
    c = np.argmin(d, axis=-1)                       # lowest code among equals
    nxt = np.minimum(c + 1, 7)
    tie = (c < 7) & (np.take_along_axis(d, nxt[..., None], -1)[..., 0] ==
                     np.take_along_axis(d, c[..., None], -1)[..., 0])
    c = np.where(tie & (c & 1 == 1), c + 1, c)
    return (c | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def mxfp4_quantize(w):
    """(packed codes uint8 [..., K/2], scales uint8 [..., K/32]) of w [..., K]."""
    w = np.asarray(w, dtype=F64)
    s = shared_exponents(w, E2M1_EMAX)
    x = np.ldexp(w.reshape(*w.shape[:-1], -1, BLOCK), -s[..., None])
    c = e2m1_encode(x).reshape(w.shape).astype(np.uint8)
    packed = c[..., 0::2] | (c[..., 1::2] << 4)
    return packed.astype(np.uint8), (s + 127).astype(np.uint8)


def mxfp4_unpack(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    c = np.empty((*p.shape[:-1], 2 * p.shape[-1]), np.uint8)
    c[..., 0::2] = p & 0xF
    c[..., 1::2] = p >> 4
    return c


def mxfp4_dequantize(packed, scales) -> np.ndarray:
    c = mxfp4_unpack(packed)
    s = np.asarray(scales, dtype=np.int64) - 127
    v = e2m1_decode(c).reshape(*c.shape[:-1], -1, BLOCK)
    return np.ldexp(v, s[..., None]).reshape(c.shape)


# ---------------------------------------------------------------------------
# Block-scaled operands on both sides (prefill experts on scaled matrix cores)
# ---------------------------------------------------------------------------

def mxfp8_round(a) -> np.ndarray:
    """An activation tensor as an MXFP8 operand: each row quantised along its
    last axis in blocks of 32 (the weights' rule) and decoded."""
    c, s = mxfp8_quantize(a)
    return mxfp8_dequantize(c, s)


def moe_mx_scaled_act(dims, x, idx, get_expert, q=mxfp8_round, gate_up=False):
    """The gate/up product of moe_mx_scaled: act[t][k] = bf16(silu(gate) * up)
    with gate, up = bf16(q(x[t]) . W13_e^T) for e = idx[t][k] (F values per
    pair; NaN rows for ids outside [0, E)). gate_up: also return gate and up."""
    from .layer import as_f64, bf, silu
    x = as_f64(x)
    idx = np.asarray(idx)
    T, K = idx.shape
    xq = q(x)
    act, gate, up = (np.full((T, K, dims.F), np.nan) for _ in range(3))
    for e in np.unique(idx):
        if not 0 <= e < dims.E:
            continue
        w13, _ = get_expert(int(e))
        tt, kk = np.nonzero(idx == e)
        u = bf(xq[tt] @ as_f64(w13).T)
        gate[tt, kk], up[tt, kk] = u[:, :dims.F], u[:, dims.F:]
        act[tt, kk] = bf(silu(u[:, :dims.F]) * u[:, dims.F:])
    return (act, gate, up) if gate_up else act


def moe_mx_scaled_down(dims, act, idx, w, get_expert, q=mxfp8_round) -> np.ndarray:
    """The down product and combine of moe_mx_scaled from given activations
    act [T][K][F]: y[t] = bf16(sum_k w[t][k] * (q(act[t][k]) . W2_e^T)) over
    the slots whose id is in [0, E)."""
    from .layer import as_f64, bf
    idx = np.asarray(idx)
    T, K = idx.shape
    acc = np.zeros((T, dims.D), F64)
    for e in np.unique(idx):
        if not 0 <= e < dims.E:
            continue
        _, w2 = get_expert(int(e))
        tt, kk = np.nonzero(idx == e)
        y = q(as_f64(act[tt, kk])) @ as_f64(w2).T
        for r, (t, k) in enumerate(zip(tt, kk)):
            acc[t] += float(w[t, k]) * y[r]
    return bf(acc)


def moe_mx_scaled(dims, x, idx, w, get_expert, q=mxfp8_round) -> np.ndarray:
    """Top-k SwiGLU experts whose products take block-scaled operands on both
    sides: the token's x enters the gate/up product as q(x) and each expert's
    activation enters the down product as q(act); get_expert(e) gives the
    (decoded) block-scaled weights (w13 [2F][D], w2 [D][F]). Otherwise the
    bf16 MoE: gate and up rounded to bf16, act = bf16(silu(gate) * up), the
    weighted combine summed wide and rounded once. q = identity gives that
    MoE on the same weights. Slots with ids outside [0, E) contribute
    nothing."""
    act = moe_mx_scaled_act(dims, x, idx, get_expert, q)
    return moe_mx_scaled_down(dims, act, idx, w, get_expert, q)
