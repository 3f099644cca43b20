"""Routed experts of a many-token step on block-scaled operands on both sides
of the products (beam_moe_swiglu_combine_mx_scaled: MXFP8 tokens and
activations times MXFP8 or MXFP4 expert weights on the scaled matrix cores).

Weights are drawn as bf16 and quantised by the library's own quantisers
(checked bit for bit against the oracle's codec elsewhere); the oracle's MoE
with both product inputs block-quantised runs on the codec's reconstruction of
the same draws. Sizes span one and several 256-row tiles per expert, ragged
tails, experts with no rows, one and several 128-deep slabs, and Beam's
expert shape (GPU).

Each call is checked in three stages, each fed what the call itself stored
for the stage before, so that every block-code decision is taken on the same
bf16 inputs on both sides: the MXFP8 copy of x (bit for bit), the activations
(to the propagated bound of their two bf16 roundings: gate/up, then act) and
the combined output from the stored activations (one rounding)."""
import numpy as np
import pytest
import torch

import moe_decoder_layer_amd as B
import synth
from beamrun import (CTL_BYTES, assert_rms_close, bf16_ulp, bits_f64, dev, host_bits, rms,
                     ws)
from oracle import mx
from test_gpu_mx import MxExperts

pytestmark = pytest.mark.gpu

CFG0 = synth.config(0).dims
BEAM = synth.config(1).dims
I16 = dict(dtype=torch.int16, device="cuda")
WBITS = {"mxfp8": 8, "mxfp4": 4}


def _dims(base, **kw):
    return synth.with_dims(synth.Config("", base), **kw).dims


def _route(dims, T, seed, skew=False):
    """Distinct experts per token; skew routes most tokens to the first experts
    (several tiles there, none on some others)."""
    g = np.random.default_rng(seed)
    if skew:
        p = np.exp(-np.arange(dims.E) / 1.5)
    else:
        p = np.ones(dims.E)
    p = p / p.sum()
    idx = np.stack([g.choice(dims.E, dims.topk, replace=False, p=p) for _ in range(T)])
    w = g.uniform(0.05, 0.6, (T, dims.topk)).astype(np.float32)
    return idx.astype(np.int32), w


def _al(n):
    return (n + 255) // 256 * 256


def _run(X, dims, T, x, idx, w):
    """y and the staged operands the call leaves at the head of its workspace:
    the pair -> row map, xq's codes and scales, act [T][topk][F] (NaN for
    pairs with a bad id)."""
    y = torch.empty((T, dims.D), **I16)
    wsb = ws(dims, B.BEAM_OP_MOE_MX_SCALED, T)
    B.beam_moe_swiglu_combine_mx_scaled(dims, T, dev(x), dev(idx), dev(w), WBITS[X.fmt], X.c13,
                                        X.s13, X.c2, X.s2, y, wsb)
    K, D, F = dims.topk, dims.D, dims.F
    P = T * K
    data = wsb[CTL_BYTES:].cpu().numpy()
    o = 0
    inv = data[o:o + 4 * P].view(np.int32).reshape(T, K)
    o += _al(4 * P)
    xq = data[o:o + T * D].reshape(T, D)
    o += _al(T * D)
    xs = data[o:o + T * D // 32].reshape(T, D // 32)
    o += _al(T * D // 32)
    act_rows = data[o:o + 2 * P * F].view(np.uint16).reshape(P, F)
    ok = (idx >= 0) & (idx < dims.E)
    act = np.full((T, K, F), np.nan)
    act[ok] = bits_f64(act_rows[inv[ok]])
    return y, dict(xq=xq, xs=xs, act=act)


def _assert_act_close(got, ref, gate, up):
    """act = bf16(silu(gate) * up) after gate, up = bf16(fp32 or fp64 sums):
    where a sum straddles a bf16 rounding boundary the two sides' gate or up
    are neighbours (one bf16 ulp apart), which moves act by up to
    |d act / d gate| ulp(gate) + |d act / d up| ulp(up), then act's own
    rounding adds one ulp. Where silu is steep relative to its value (gate
    large and negative) that exceeds a fixed number of act ulps. Every element
    within max(1e-2 rms(ref), that bound); the RMS of the error within
    1e-2 rms(ref)."""
    sg = 1.0 / (1.0 + np.exp(-gate))
    d_gate = np.abs(sg * (1.0 + gate * (1.0 - sg)) * up)
    d_up = np.abs(gate * sg)
    bound = (bf16_ulp(np.maximum(np.abs(got), np.abs(ref))) + d_gate * bf16_ulp(gate)
             + d_up * bf16_ulp(up)) * 1.001
    err = np.abs(got - ref)
    r = rms(ref)
    assert np.all(np.isfinite(got)), "act: non-finite GPU values"
    bad = err > np.maximum(1e-2 * r, bound)
    assert not np.any(bad), (f"act: {int(bad.sum())} of {err.size} elements beyond the bound; "
                             f"worst |err| {err.max():.3e}, rms {r:.3e}")
    assert rms(got - ref) <= 1e-2 * r


def _check(X, dims, x, idx, w, y, st):
    """Stage by stage against the oracle (see the module's docstring)."""
    c_ref, s_ref = mx.mxfp8_quantize(bits_f64(x))
    np.testing.assert_array_equal(st["xs"], s_ref)
    np.testing.assert_array_equal(st["xq"], c_ref)
    ok = (idx >= 0) & (idx < dims.E)
    act_ref, gate, up = mx.moe_mx_scaled_act(dims, x, idx, X.expert, gate_up=True)
    _assert_act_close(st["act"][ok], act_ref[ok], gate[ok], up[ok])
    got = bits_f64(host_bits(y))
    assert_rms_close(got, mx.moe_mx_scaled_down(dims, st["act"], idx, w, X.expert), "y2")
    return got


CASES = [
    ("one_slab", dict(D=128, F=128, E=4, topk=2), 37, False),
    ("small", dict(D=256, F=128, E=8, topk=2), 40, False),
    ("tiles", dict(D=512, F=256, E=16, topk=4), 300, False),
    ("skew", dict(D=384, F=384, E=6, topk=2), 700, True),
    ("one_token", dict(D=256, F=256, E=8, topk=3), 1, False),
]


@pytest.mark.parametrize("name,kw,T,skew", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_moe_mx_scaled(fmt, name, kw, T, skew):
    dims = _dims(CFG0, n_group=1, topk_group=1, **kw)
    X = MxExperts(fmt, dims, "sc_" + name)
    x = synth.make_h((T, dims.D), 7, "mxsx", name, T)
    idx, w = _route(dims, T, 5 + T, skew)
    y, st = _run(X, dims, T, x, idx, w)
    B.beam_check()
    got = _check(X, dims, x, idx, w, y, st)
    if name == "tiles":
        # end to end the operand rounding is visible: the same MoE without it
        # is several times further away than the oracle's scaled MoE
        plain = mx.moe_mx_scaled(dims, x, idx, w, X.expert, q=lambda a: a)
        ref = mx.moe_mx_scaled(dims, x, idx, w, X.expert)
        assert rms(got - ref) * 4 < rms(got - plain)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_moe_mx_scaled_beam_shape(fmt):
    """Beam's expert shape (D 5,120, F 2,560), two experts, 300 tokens routed
    to both: 600 rows, three tiles per expert with a ragged last one."""
    dims = _dims(BEAM, E=2, topk=2, n_group=1, topk_group=1)
    X = MxExperts(fmt, dims, "sc_beam", device_draw=True)
    T = 300
    x = synth.make_h((T, dims.D), 7, "mxsbx")
    g = np.random.default_rng(2)
    idx = np.stack([g.permutation(2) for _ in range(T)]).astype(np.int32)
    w = g.uniform(0.05, 0.6, (T, 2)).astype(np.float32)
    y, st = _run(X, dims, T, x, idx, w)
    B.beam_check()
    _check(X, dims, x, idx, w, y, st)


def test_moe_mx_scaled_bad_expert_id_is_flagged():
    dims = _dims(CFG0, D=256, F=128, E=8, topk=2, n_group=1, topk_group=1)
    X = MxExperts("mxfp8", dims, "sc_bad")
    T = 5
    x = synth.make_h((T, dims.D), 7, "mxsbad")
    idx = np.array([[1, 2], [dims.E, 3], [4, -1], [0, 7], [6, 5]], np.int32)
    w = np.full((T, 2), 0.5, np.float32)
    y, st = _run(X, dims, T, x, idx, w)
    with pytest.raises(B.BeamError) as e:
        B.beam_check()
    assert e.value.code == -8
    B.beam_check()
    _check(X, dims, x, idx, w, y, st)   # the bad slots contribute nothing


def test_moe_mx_scaled_rejections():
    dims = _dims(CFG0, D=256, F=128, E=8, topk=2, n_group=1, topk_group=1)
    X = MxExperts("mxfp8", dims, "sc_rej")
    T = 4
    x = torch.zeros((T, dims.D), **I16)
    idx = torch.zeros((T, 2), dtype=torch.int32, device="cuda")
    w = torch.zeros((T, 2), dtype=torch.float32, device="cuda")
    y = torch.empty((T, dims.D), **I16)
    wsb = ws(dims, B.BEAM_OP_MOE_MX_SCALED, T)
    with pytest.raises(B.BeamError) as e:        # neither MXFP8 nor MXFP4
        B.beam_moe_swiglu_combine_mx_scaled(dims, T, x, idx, w, 6, X.c13, X.s13, X.c2, X.s2,
                                            y, wsb)
    assert e.value.code == -2
    odd = _dims(dims, D=288)
    with pytest.raises(B.BeamError) as e:        # D not a multiple of the slab depth
        B.beam_moe_swiglu_combine_mx_scaled(odd, T, x, idx, w, 8, X.c13, X.s13, X.c2, X.s2,
                                            y, wsb)
    assert e.value.code == -3
    with pytest.raises(B.BeamError) as e:        # workspace too small
        B.beam_moe_swiglu_combine_mx_scaled(dims, T, x, idx, w, 8, X.c13, X.s13, X.c2, X.s2,
                                            y, wsb[:512])
    assert e.value.code == -5


def test_moe_mx_scaled_full_size():
    """The benchmark's prefill MoE shape: 16,384 tokens, top-8 of all 256
    experts of Beam's size (uniform routing), MXFP8 weights. Sampled: the
    MXFP8 copy of x bit for bit on 512 tokens; one token's eight activation
    rows and its output row stage by stage against the oracle; every output
    row finite and no device flag."""
    dims = BEAM
    T = 8 * 2048
    X = MxExperts("mxfp8", dims, "sc_full", device_draw=True)
    x = synth.make_h((T, dims.D), 7, "mxsfull")
    g = np.random.default_rng(31)
    idx = np.argsort(g.random((T, dims.E)), axis=1)[:, :dims.topk].astype(np.int32)
    w = g.uniform(0.05, 0.6, (T, dims.topk)).astype(np.float32)
    K, D, F = dims.topk, dims.D, dims.F
    P = T * K
    y = torch.empty((T, D), **I16)
    wsb = ws(dims, B.BEAM_OP_MOE_MX_SCALED, T)
    B.beam_moe_swiglu_combine_mx_scaled(dims, T, dev(x), dev(idx), dev(w), 8, X.c13, X.s13, X.c2,
                                        X.s2, y, wsb)
    B.beam_check()
    yb = y.view(torch.bfloat16)
    assert bool(torch.isfinite(yb.float()).all()), "non-finite output rows"
    # staged operands at the head of the workspace (see _run)
    data = wsb[CTL_BYTES:]
    o = 0
    inv = data[o:o + 4 * P].view(torch.int32).view(T, K)
    o += _al(4 * P)
    xq = data[o:o + T * D].view(T, D)
    o += _al(T * D)
    xs = data[o:o + T * D // 32].view(T, D // 32)
    o += _al(T * D // 32)
    act_rows = data[o:o + 2 * P * F].view(torch.int16).view(P, F)
    rows = np.sort(g.choice(T, 512, replace=False))
    c_ref, s_ref = mx.mxfp8_quantize(bits_f64(x[rows]))
    np.testing.assert_array_equal(xs[rows].cpu().numpy(), s_ref)
    np.testing.assert_array_equal(xq[rows].cpu().numpy(), c_ref)
    t = int(rows[len(rows) // 2])
    act = np.full((1, K, F), np.nan)
    act[0] = bits_f64(host_bits(act_rows[inv[t].long()]))
    xt, it, wt = x[t:t + 1], idx[t:t + 1], w[t:t + 1]
    act_ref, gate, up = mx.moe_mx_scaled_act(dims, xt, it, X.expert, gate_up=True)
    _assert_act_close(act[0], act_ref[0], gate[0], up[0])
    assert_rms_close(bits_f64(host_bits(y[t:t + 1])),
                     mx.moe_mx_scaled_down(dims, act, it, wt, X.expert), "y2 full size")
