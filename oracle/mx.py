"""MXFP8 block quantisation of expert weights, written from the OCP
Microscaling (MX) format definition (test infrastructure only; see
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

w / X is exact (X is a power of two inside the float64 range), so the only
rounding is the E4M3 encoding, the same in any precision that holds w.
"""
from __future__ import annotations

import numpy as np

from .numerics import e4m3_decode, e4m3_encode

F64 = np.float64
BLOCK = 32
E4M3_EMAX = 8


def shared_exponents(w) -> np.ndarray:
    """Scale exponent s of every 32-element block along the last axis."""
    w = np.asarray(w, dtype=F64)
    assert w.shape[-1] % BLOCK == 0, "K must be a multiple of 32"
    amax = np.abs(w.reshape(*w.shape[:-1], w.shape[-1] // BLOCK, BLOCK)).max(axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))   # 2**(e-1) <= amax < 2**e
    s = (e - 1) - E4M3_EMAX
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
