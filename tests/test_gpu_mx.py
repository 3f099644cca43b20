"""Block-scaled (MXFP8 and MXFP4) expert weights at decode steps.

The quantisers must agree bit for bit with the oracle's codecs (per 32 weights
along K a shared exponent floor(log2 amax) - 8 with e4m3fn codes, or
floor(log2 amax) - 2 with nibble-packed e2m1 codes; codes rounded to nearest
even and saturated). The expert calls are compared, to the same bar as the
bf16 expert call, with the oracle's MoE run on the weights the oracle's own
codec reconstructs from the bf16 draws."""
import numpy as np
import pytest
import torch

import moe_decoder_layer_amd as B
import synth
from beamrun import assert_rms_close, bits_f64, dev, host_bits, ws
from oracle import layer as L
from oracle import mx

pytestmark = pytest.mark.gpu

CFG0 = synth.config(0).dims
BEAM = synth.config(1).dims
U8 = dict(dtype=torch.uint8, device="cuda")
I16 = dict(dtype=torch.int16, device="cuda")


def _dims(base, **kw):
    return synth.with_dims(synth.Config("", base), **kw).dims


FMTS = ["mxfp8", "mxfp4"]
ORACLE = {"mxfp8": (mx.mxfp8_quantize, mx.mxfp8_dequantize),
          "mxfp4": (mx.mxfp4_quantize, mx.mxfp4_dequantize)}


def _quantize(fmt, w, rows, K):
    codes = torch.empty((rows, K if fmt == "mxfp8" else K // 2), **U8)
    scales = torch.empty((rows, K // 32), **U8)
    getattr(B, f"beam_{fmt}_quantize")(w, rows, K, codes, scales)
    return codes, scales


def _special_rows(K, seed):
    """bf16 bit rows that reach every branch of the codec: an all-zero block,
    signed zeros, bf16 subnormals, huge magnitudes, blocks whose largest value
    saturates (amax / 2^s >= 448) and small values next to a large one (e4m3
    subnormals and underflow to zero)."""
    g = np.random.default_rng(seed)
    rows = []
    r = np.zeros(K, np.uint16)
    r[32:64] = 0x8000                                        # -0 block
    r[64:96] = g.integers(1, 0x80, r[64:96].size)            # positive subnormals
    rows.append(r)
    r = synth.normal_bf16((K,), 1.0, seed, "mx_special", 1)
    r[::32] = 0x7f70                                          # 2^127 * 1.875 (saturates)
    rows.append(r)
    r = synth.normal_bf16((K,), 1e-4, seed, "mx_special", 2)
    r[5::32] = 0x4500                                        # 2048 beside 1e-4 values
    rows.append(r)
    r = synth.normal_bf16((K,), 1.0, seed, "mx_special", 3)
    r[7::32] = 0xc3f8                                        # -496: amax/2^s = 496 -> 448
    r[9::32] = 0x0040                                        # subnormal in a normal block
    rows.append(r)
    r = (g.integers(0, 0x10000, K)).astype(np.uint16)
    r = np.where((r & 0x7f80) == 0x7f80, r & 0xbfff, r)      # random finite bit patterns
    rows.append(r.astype(np.uint16))
    return np.stack(rows)


@pytest.mark.parametrize("rows,K", [(1, 32), (37, 96), (300, 5120), (2 * 512 + 3, 2048)])
@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_bit_exact(fmt, rows, K):
    w = synth.normal_bf16((rows, K), 0.02, 0, "mx_q", rows, K)
    sp = _special_rows(K, rows)
    w[-min(rows, len(sp)):] = sp[:min(rows, len(sp))]
    codes, scales = _quantize(fmt, dev(w), rows, K)
    B.beam_check()
    c_ref, s_ref = ORACLE[fmt][0](bits_f64(w))
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_rows_zero_is_a_no_op(fmt):
    codes = torch.full((1, 32), 7, **U8)
    getattr(B, f"beam_{fmt}_quantize")(torch.zeros((1, 32), **I16), 0, 32, codes,
                                       torch.empty((1, 1), **U8))
    B.beam_check()
    assert int(codes.sum()) == 7 * 32


class MxExperts:
    """Expert weights drawn as bf16, quantised on the device by the library;
    the oracle side quantises the same bf16 draws with its own codec."""

    def __init__(self, fmt, dims, tag, device_draw=False):
        self.fmt = fmt
        E, F, D = dims.E, dims.F, dims.D
        if device_draw:
            self.w13 = synth.torch_normal_bf16((E, 2 * F, D), 0.02, 0, "mx_w13", tag)
            self.w2 = synth.torch_normal_bf16((E, D, F), 0.02, 0, "mx_w2", tag)
        else:
            self.w13 = dev(synth.normal_bf16((E, 2 * F, D), 0.02, 0, "mx_w13", tag))
            self.w2 = dev(synth.normal_bf16((E, D, F), 0.02, 0, "mx_w2", tag))
        self.c13, self.s13 = _quantize(fmt, self.w13, E * 2 * F, D)
        self.c2, self.s2 = _quantize(fmt, self.w2, E * D, F)
        self._ref = {}

    def expert(self, e):
        """Oracle weights of expert e: the codec's reconstruction of the draws."""
        if e not in self._ref:
            q, dq = ORACLE[self.fmt]
            w13 = dq(*q(bits_f64(host_bits(self.w13[e]))))
            w2 = dq(*q(bits_f64(host_bits(self.w2[e]))))
            self._ref[e] = (w13, w2)
        return self._ref[e]

    def run(self, dims, T, x, idx, w):
        y = torch.empty((T, dims.D), **I16)
        call = getattr(B, f"beam_moe_swiglu_combine_{self.fmt}")
        call(dims, T, dev(x), dev(idx), dev(w), self.c13, self.s13, self.c2, self.s2, y,
             ws(dims, B.BEAM_OP_MOE, T))
        return y


def _route(dims, T, seed):
    g = np.random.default_rng(seed)
    idx = np.stack([g.choice(dims.E, dims.topk, replace=False) for _ in range(T)]).astype(np.int32)
    w = g.uniform(0.05, 0.6, (T, dims.topk)).astype(np.float32)
    return idx, w


# D and F chosen so that both GEMVs take their one-chunk and many-chunk forms,
# with full and with partly masked lanes (16-code chunks), and with the scales
# read as words (K a multiple of 128) or byte by byte
SMALL = [
    ("cfg0", {}),
    ("ragged", dict(D=1056, F=96, E=6, topk=3)),
    ("wide_f", dict(D=288, F=2080, E=5, topk=2)),
    ("words", dict(D=512, F=256, E=4, topk=2)),
    ("wide_d", dict(D=2080, F=64, E=4, topk=2)),
]


@pytest.mark.parametrize("T", [1, 3, 4])
@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("fmt", FMTS)
def test_moe_mx(fmt, name, kw, T):
    dims = _dims(CFG0, n_group=1, topk_group=1, **kw) if kw else CFG0
    X = MxExperts(fmt, dims, name)
    x = synth.make_h((T, dims.D), 7, "mxx", name, T)
    idx, w = _route(dims, T, 11 + T)
    y = X.run(dims, T, x, idx, w)
    B.beam_check()
    assert_rms_close(bits_f64(host_bits(y)), L.moe(dims, x, idx, w, X.expert), "y2")


@pytest.mark.parametrize("fmt", FMTS)
def test_moe_mx_beam_shape(fmt):
    """Beam's expert shape (D 5,120, F 2,560): two experts, two tokens routed
    to both in opposite order with different weights."""
    dims = _dims(BEAM, E=2, topk=2, n_group=1, topk_group=1)
    X = MxExperts(fmt, dims, "beam", device_draw=True)
    T = 2
    x = synth.make_h((T, dims.D), 7, "mxbx")
    idx = np.array([[1, 0], [0, 1]], np.int32)
    w = np.array([[0.55, 0.2], [0.35, 0.125]], np.float32)
    y = X.run(dims, T, x, idx, w)
    B.beam_check()
    assert_rms_close(bits_f64(host_bits(y)), L.moe(dims, x, idx, w, X.expert), "y2")


@pytest.mark.parametrize("fmt", FMTS)
def test_moe_mx_bad_expert_id_is_flagged(fmt):
    dims = CFG0
    X = MxExperts(fmt, dims, "bad")
    x = synth.make_h((1, dims.D), 7, "mxbad")
    idx = np.array([[1, 2, dims.E, 3]], np.int32)
    w = np.full((1, 4), 0.5, np.float32)
    y = X.run(dims, 1, x, idx, w)
    with pytest.raises(B.BeamError) as e:
        B.beam_check()
    assert e.value.code == -8
    B.beam_check()
    ref = L.moe(dims, x, np.array([[1, 2, 3]]), w[:, :3], X.expert)
    assert_rms_close(bits_f64(host_bits(y)), ref, "y2 without the bad slot")


@pytest.mark.parametrize("fmt", FMTS)
def test_moe_mx_rejects_prefill_sizes(fmt):
    dims = CFG0
    X = MxExperts(fmt, dims, "big")
    T = 5
    x = torch.zeros((T, dims.D), **I16)
    idx = torch.zeros((T, dims.topk), dtype=torch.int32, device="cuda")
    w = torch.zeros((T, dims.topk), dtype=torch.float32, device="cuda")
    y = torch.empty((T, dims.D), **I16)
    with pytest.raises(B.BeamError) as e:
        getattr(B, f"beam_moe_swiglu_combine_{fmt}")(dims, T, x, idx, w, X.c13, X.s13, X.c2,
                                                     X.s2, y, ws(dims, B.BEAM_OP_MOE, T))
    assert e.value.code == -3
