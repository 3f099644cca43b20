"""Whole-layer parity of the HIP path (the eight C calls in order) against the
oracle: every stage fed the GPU's upstream tensors, then the layer end to end
from the same inputs (GPU)."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from beamrun import (Cache, Params, assert_rms_close, bf16_ulp, bits_f64, check_routing,
                     code_pos, dev, host_bits, rms, run_layer)
from oracle import layer as L
from oracle.numerics import e4m3_quantize, f64_to_bf16_bits, round_bf16

pytestmark = pytest.mark.gpu


def check_stages(dims, P: Params, cache: Cache, g, pos, seq, mode, n, ffn, sink=None,
                 sandwich=True):
    """Each stage of the GPU layer against the oracle run on the GPU's inputs
    (sandwich False: the pre-norm, plain-residual layer form)."""
    eps = dims.eps
    _, x_ref = L.boundary(None, g["h_in"], None, P.np("w_attn_pre"), 0, eps)
    assert_rms_close(bits_f64(g["x"]), x_ref, "x")
    qkvg = L.qkvg_projection(g["x"], P.np("w_qkvg"))
    nqkv = (dims.Hq + 2 * dims.Hkv) * dims.d
    assert_rms_close(bits_f64(g["qkv"]), qkvg[:, :nqkv], "qkv projection")
    # the per-head stage is fed the GPU's stored projection
    q, k, v, _ = L.split_qkvg(dims, np.concatenate([bits_f64(g["qkv"]), qkvg[:, nqkv:]], 1))
    gg = qkvg[:, nqkv:nqkv + dims.G]
    qn, kn = L.qk_norm_position(dims, q, k, pos, mode, P.np("w_qnorm"), P.np("w_knorm"))
    assert_rms_close(bits_f64(g["q"]), round_bf16(qn), "q")
    if dims.G:
        assert_rms_close(bits_f64(g["g"]), gg, "g")
    K = cache.K.cpu().numpy()
    Vt = cache.V.cpu().numpy()
    for t in range(len(pos)):
        s, p = seq[t], pos[t]
        if cache.kv == "bf16":
            assert_rms_close(bits_f64(K[s, :, p].view(np.uint16)), round_bf16(kn[t]), "k write")
            assert_rms_close(bits_f64(Vt[s, :, :, p].view(np.uint16)), v[t], "v write")
        else:
            assert np.max(np.abs(code_pos(K[s, :, p]) -
                                 code_pos(e4m3_quantize(kn[t], cache.k_scale)))) <= 1
            assert np.max(np.abs(code_pos(Vt[s, :, :, p]) -
                                 code_pos(e4m3_quantize(v[t], cache.v_scale)))) <= 1
    mp = int(np.max(pos))
    o_ref = L.attention(dims, bits_f64(g["q"]), pos, seq, cache.oracle(mp + 1), mode, sink)
    T = len(pos)
    if g.get("z") is not None:
        # fused call: the gated output against the oracle's gate over its
        # attention (two rounding points: o, then z)
        z_ref = (L.output_gate(dims, o_ref, bits_f64(g["g"]), P.np("b_gate")) if dims.G
                 else o_ref.reshape(T, -1))
        assert_rms_close(bits_f64(g["z"]), z_ref, "z fused", ulps=2)
        z = bits_f64(g["z"])
    else:
        assert_rms_close(bits_f64(g["o"]), o_ref, "o")
        if dims.G:
            z = L.output_gate(dims, bits_f64(g["o"]), bits_f64(g["g"]), P.np("b_gate"))
        else:
            z = bits_f64(g["o"]).reshape(T, -1)
    assert_rms_close(bits_f64(g["y"]), L.o_proj(z, P.np("w_o")), "y")
    w_post, n_a = (P.np("w_attn_post"), n) if sandwich else (None, 0)
    hm, _ = L.boundary(g["y"], g["h_in"], w_post, P.np("w_ffn_pre"), n_a, eps)
    assert_rms_close(bits_f64(g["h_mid"]), hm, "h_mid")
    _, x2 = L.boundary(None, g["h_mid"], None, P.np("w_ffn_pre"), 0, eps)
    assert_rms_close(bits_f64(g["x2"]), x2, "x2")
    if ffn == "moe":
        check_routing(dims, g["x2"], P, g["idx"], g["w"], g["logits"], "router")
        shared = (P.np("shared_w13"), P.np("shared_w2")) if dims.shared else None
        y2 = L.moe(dims, g["x2"], g["idx"], g["w"], P.expert, shared)
    else:
        y2 = L.dense_ffn(g["x2"], P.np("dense_w13"), P.np("dense_w2"), dims.Fd)
    assert_rms_close(bits_f64(g["y2"]), y2, "y2")
    w_post, n_f = (P.np("w_ffn_post"), n + 1) if sandwich else (None, 0)
    ho, _ = L.boundary(g["y2"], g["h_mid"], w_post, P.np("w_next_pre"), n_f, eps)
    assert_rms_close(bits_f64(g["h_out"]), ho, "h_out")
    _, xn = L.boundary(None, g["h_out"], None, P.np("w_next_pre"), 0, eps)
    assert_rms_close(bits_f64(g["x_next"]), xn, "x_next")
    assert T == len(g["h_out"])


def check_end_to_end(dims, P, ocache, g, h, pos, seq, mode, n, ffn, experts=None,
                     sandwich=True):
    """The oracle's whole layer from the same inputs; near-tie tokens replay
    the GPU's routing."""
    od = P.oracle_dict(experts=experts is None and ffn == "moe")
    r = L.layer_forward(dims, od, h, pos, seq, ocache.copy(), mode, n, ffn=ffn,
                        get_expert=experts, sandwich=sandwich)
    if ffn == "moe":
        tie = (r["group_margin"] <= 1e-4) | (r["expert_margin"] <= 1e-4)
        same = np.array([set(a) == set(b) for a, b in zip(r["idx"].tolist(), g["idx"].tolist())])
        if not np.all(same):
            assert np.all(same | tie), "routing differs on a token without a near tie"
            r = L.layer_forward(dims, od, h, pos, seq, ocache.copy(), mode, n, ffn=ffn,
                                get_expert=experts, route_override=g["idx"], sandwich=sandwich)
    check_h_out_e2e(g, r)
    check_x_next_e2e(dims, P, g, r)


def check_h_out_e2e(g, r):
    """h_out = bf16(h_mid + y2), with h_mid and y2 themselves bf16: where the
    GPU's fp32 value and the oracle's float64 value straddle a rounding
    boundary at any of these three points, the results differ by one ulp of
    that tensor at that element (h_mid's ulp can be twice h_out's when the
    sum drops a binade). Every element stays within max(1e-2 * rms, the sum
    of those three ulps), and the error RMS within 1e-2 * rms."""
    got, ref = bits_f64(g["h_out"]), np.asarray(r["h_out"], np.float64)
    assert np.all(np.isfinite(got)), "h_out (end to end): non-finite GPU values"

    def ulp(k):
        a, b = bits_f64(g[k]), np.asarray(r[k], np.float64)
        return bf16_ulp(np.maximum(np.abs(a), np.abs(b)))

    allow = (ulp("h_out") + ulp("h_mid") + ulp("y2")) * 1.0000001
    err = np.abs(got - ref)
    bad = err > np.maximum(1e-2 * rms(ref), allow)
    assert not np.any(bad), (f"h_out (end to end): {int(bad.sum())} of {err.size} elements beyond "
                             f"max(0.01*rms, rounding allowance); worst |err| {err.max():.3e}")
    assert rms(err) <= 1e-2 * rms(ref), "h_out (end to end): error rms"


def check_x_next_e2e(dims, P, g, r):
    """x_next = rms(h_out) * w: the h_out bar carried through the norm. An h_out
    error e_i becomes e_i * w_i / rms(h_out) in x_next, plus x_next's own
    rounding (one ulp); the error RMS must stay within 1e-2 * rms(x_next)."""
    h_ref, x_ref = r["h_out"], r["x_next"]
    x_got = bits_f64(g["x_next"])
    w = bits_f64(P.np("w_next_pre"))
    inv = 1.0 / np.sqrt(np.mean(h_ref * h_ref, axis=-1, keepdims=True) + dims.eps)
    tol_h = np.maximum(1e-2 * rms(h_ref), 2 * bf16_ulp(h_ref))
    bound = tol_h * inv * w + bf16_ulp(x_ref) * 1.0000001
    err = np.abs(x_got - x_ref)
    assert np.all(err <= bound), f"x_next (end to end): worst excess {np.max(err - bound):.3e}"
    assert rms(err) <= 1e-2 * rms(x_ref), "x_next (end to end): error rms"


def _tiny(mode, kv, T, ffn="moe", S=1):
    cfg = synth.config(0)
    dims, ex = cfg.dims, cfg.extra
    P = Params(dims, 0, ex["layer"], moe=(ffn == "moe"), dense=(ffn == "dense"))
    Kp, Vp, ks, vs = synth.torch_kv_prior(dims, S, ex["ctx"], kv, 0, ex["layer"])
    cache = Cache(dims, S, ex["Lmax"], kv, ks, vs)
    cache.fill_prior(Kp, Vp)
    if T == 1:
        pos = np.array([ex["ctx"]], np.int32)
    else:
        pos = np.concatenate([np.arange(ex["ctx"], ex["ctx"] + T // S) for _ in range(S)])
        pos = pos.astype(np.int32)
    seq = np.repeat(np.arange(S), len(pos) // S).astype(np.int32)
    h = synth.make_h((len(pos), dims.D), 0, "tiny", mode, kv, T)
    return dims, P, cache, h, pos, seq, ex["n"]


@pytest.mark.parametrize("mode", ["swa", "nope"])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("T,fused", [(1, False), (1, True), (32, False)])
def test_tiny_layer(mode, kv, T, fused):
    dims, P, cache, h, pos, seq, n = _tiny(mode, kv, T)
    ocache = cache.oracle()                     # prior only, before the layer writes
    g = run_layer(dims, P, cache, h, pos, seq, mode, n, fused=fused)
    check_stages(dims, P, cache, g, pos, seq, mode, n, "moe")
    # positions beyond the prior held NaN patterns in the GPU cache: the oracle's zeros
    # stand in for "never read"
    check_end_to_end(dims, P, ocache, g, h, pos, seq, mode, n, "moe")


def test_tiny_layer_two_sequences_dense_ffn():
    dims, P, cache, h, pos, seq, n = _tiny("swa", "bf16", 32, ffn="dense", S=2)
    ocache = cache.oracle()
    g = run_layer(dims, P, cache, h, pos, seq, "swa", n, ffn="dense")
    check_stages(dims, P, cache, g, pos, seq, "swa", n, "dense")
    check_end_to_end(dims, P, ocache, g, h, pos, seq, "swa", n, "dense")


def test_tiny_layer_deterministic():
    outs = []
    for _ in range(2):
        dims, P, cache, h, pos, seq, n = _tiny("nope", "fp8", 32)
        outs.append(run_layer(dims, P, cache, h, pos, seq, "nope", n))
    for k in ("q", "o", "y", "x2", "y2", "h_out", "x_next", "idx", "w", "logits"):
        np.testing.assert_array_equal(outs[0][k], outs[1][k], err_msg=k)


def test_chunked_prefill_equals_decodes():
    """prefill(8) then 4 decodes == prefill(12) on the GPU (same maths per token)."""
    dims, P, cache, h, pos, seq, n = _tiny("nope", "bf16", 12)
    c2 = cache.clone()
    full = run_layer(dims, P, cache, h, pos, seq, "nope", n)
    a = run_layer(dims, P, c2, h[:8], pos[:8], seq[:8], "nope", n)
    parts = [a["h_out"]]
    for i in range(8, 12):
        parts.append(run_layer(dims, P, c2, h[i:i + 1], pos[i:i + 1], seq[i:i + 1], "nope",
                               n)["h_out"])
    got = bits_f64(np.concatenate(parts))
    assert_rms_close(got, bits_f64(full["h_out"]), "chunked vs whole")


# ------------------------------------------------------------------ full size
_FULL = {}


def _config(i):
    """Config i, or "1m": the NoPE fp8 decode at a 2^20-token context (2 GiB
    of fp8 KV for the layer; nine such layers make the pages' 18 GiB)."""
    if i == "1m":
        cfg = synth.config(2)
        ctx = 1 << 20
        return dataclasses.replace(cfg, extra={**cfg.extra, "pos": ctx, "Lmax": ctx + 64})
    return synth.config(i)


def _full(i):
    """Beam layer at full size: all 256 experts (20 GB) drawn on the device."""
    if i not in _FULL:
        _FULL.clear()
        torch.cuda.empty_cache()
        cfg = _config(i)
        dims, ex = cfg.dims, cfg.extra
        P = Params(dims, 0, ex["layer"], moe=True, device_draw=True)
        Kp, Vp, ks, vs = synth.torch_kv_prior(dims, 1, ex["pos"], ex["kv"], 0, ex["layer"])
        cache = Cache(dims, 1, ex["Lmax"], ex["kv"], ks, vs)
        cache.fill_prior(Kp, Vp)
        del Kp, Vp
        _FULL[i] = (cfg, P, cache)
    return _FULL[i]


@pytest.mark.parametrize("i,fused", [(1, False), (1, True), (2, False), (2, True),
                                     pytest.param("1m", True, marks=pytest.mark.timeout(900))])
def test_full_size_decode(i, fused):
    """Full size in the benchmark's launch configuration (fused: the one-token
    fused attention call and o_proj alone, as the benchmark's decode legs)."""
    cfg, P, cache, = _full(i)
    dims, ex = cfg.dims, cfg.extra
    pos = np.array([ex["pos"]], np.int32)
    seq = np.zeros(1, np.int32)
    h = synth.make_h((1, dims.D), 0, "full", i)
    before = cache.clone()
    g = run_layer(dims, P, cache, h, pos, seq, ex["mode"], ex["n"], fused=fused)
    check_stages(dims, P, cache, g, pos, seq, ex["mode"], ex["n"], "moe")
    ocache = before.oracle(ex["pos"] + 1)
    check_end_to_end(dims, P, ocache, g, h, pos, seq, ex["mode"], ex["n"], "moe",
                     experts=P.expert)
