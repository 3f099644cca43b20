"""Decode stack (beam_decode_stack): one token through consecutive layers of
the model's schedule (beam_layer_kind: sliding-window layers on ring caches,
NoPE layers on full caches, dense then MoE FFNs), on a small configuration of
seven layers (layers 5 and 6 NoPE, 0-2 dense).

Each layer run alone through the stack call is bit-identical to the
single-layer calls composed by the test harness (run_layer, fused attention
half), whose outputs are checked end to end against the oracle's layer; the
seven layers in one call are bit-identical to the layers called one by one,
over three consecutive decode steps (GPU)."""
import numpy as np
import pytest
import torch

import moe_decoder_layer_amd as B
import synth
from beamrun import Cache, Params, dev, host_bits, rope_table, run_layer, ws
from test_gpu_layer import check_end_to_end
from test_gpu_ring import Ring, _ring_of

pytestmark = pytest.mark.gpu

CFG0 = synth.config(0).dims   # window 16
N, P0, LMAX, SLOTS = 7, 300, 1024, 64
I16 = dict(dtype=torch.int16, device="cuda")


def _model(kv):
    """Per layer: kind, Params (w_next_pre = the next layer's w_attn_pre), the
    linear cache holding the prior and the cache the stack uses (a ring on
    sliding-window layers)."""
    dims = CFG0
    out = []
    for l in range(N):
        mode, dense = B.beam_layer_kind(l, N)
        P = Params(dims, 11, l, moe=not dense, dense=bool(dense))
        Kp, Vp, ks, vs = synth.torch_kv_prior(dims, 1, P0, kv, 11, l)
        lin = Cache(dims, 1, LMAX, kv, ks, vs)
        lin.fill_prior(Kp, Vp)
        use = _ring_of(lin, SLOTS, [P0]) if mode == B.BEAM_SWA_ROPE else lin.clone()
        if mode == B.BEAM_SWA_ROPE:
            use.npos = LMAX
        out.append(dict(mode=mode, dense=dense, P=P, lin=lin, cache=use))
    for l in range(N - 1):   # the stack's next-layer pre-norm
        nxt = out[l + 1]["P"]
        out[l]["P"].t["w_next_pre"] = nxt.t["w_attn_pre"]
        out[l]["P"]._np["w_next_pre"] = nxt._np["w_attn_pre"]
    return dims, out


def _layer_struct(m, cache):
    P = m["P"]
    w = dict(P.t)
    if m["dense"]:
        w["w13"], w["w2"] = P.t["dense_w13"], P.t["dense_w2"]
    return B.stack_layer(m["mode"], m["dense"], w, cache.struct())


def _stack_ws(dims):
    n = B.beam_decode_stack_workspace(dims, dims.Fd, LMAX)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_stack_layers_match_single_layer_calls_and_oracle(kv):
    dims, model = _model(kv)
    rope = rope_table(LMAX, dims.d, dims.theta)
    pos, seq = np.array([P0], np.int32), np.array([0], np.int32)
    pt, st = dev(pos), dev(seq)
    wsb = _stack_ws(dims)
    h = dev(synth.make_h((1, dims.D), 4, "stack_h", kv))
    x = torch.empty((1, dims.D), **I16)
    for l, m in enumerate(model):
        mode = "swa" if m["mode"] == B.BEAM_SWA_ROPE else "nope"
        ffn = "dense" if m["dense"] else "moe"
        h_in = host_bits(h)
        ref_cache = m["cache"].clone()
        if isinstance(m["cache"], Ring):
            ref_cache = _ring_of(m["lin"], SLOTS, [P0])
            ref_cache.npos = LMAX
        ocache = m["lin"].oracle(P0 + 1)
        g = run_layer(dims, m["P"], ref_cache, h_in, pos, seq, mode, 2 * l + 1, ffn=ffn,
                      rope=rope, fused=True)
        B.beam_decode_stack(dims, dims.Fd, l, [_layer_struct(m, m["cache"])],
                            m["P"].t["w_next_pre"], h, x, pt, st, rope, P0, wsb)
        B.beam_check()
        assert np.array_equal(host_bits(h), g["h_out"]), f"layer {l}: h differs from run_layer"
        assert np.array_equal(host_bits(x), g["x_next"]), f"layer {l}: x differs from run_layer"
        assert torch.equal(m["cache"].K, ref_cache.K) and torch.equal(m["cache"].V, ref_cache.V)
        check_end_to_end(dims, m["P"], ocache, g, h_in, pos, seq, mode, 2 * l + 1, ffn)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_stack_one_call_equals_layer_by_layer(kv):
    dims, model = _model(kv)
    rope = rope_table(LMAX, dims.d, dims.theta)
    seq = dev(np.array([0], np.int32))
    w_final = model[-1]["P"].t["w_next_pre"]
    caches_a = [m["cache"] for m in model]
    caches_b = [c.clone() for c in caches_a]
    for c, m in zip(caches_b, model):
        if isinstance(m["cache"], Ring):
            c.__class__, c.npos = Ring, m["cache"].npos
    ha = dev(synth.make_h((1, dims.D), 5, "stack_h2", kv))
    hb = ha.clone()
    xa, xb = torch.empty((1, dims.D), **I16), torch.empty((1, dims.D), **I16)
    wsa, wsb = _stack_ws(dims), _stack_ws(dims)
    for step in range(3):
        p = P0 + step
        pt = dev(np.array([p], np.int32))
        B.beam_decode_stack(dims, dims.Fd, 0, [_layer_struct(m, c) for m, c in zip(model, caches_a)],
                            w_final, ha, xa, pt, seq, rope, p, wsa)
        for l, (m, c) in enumerate(zip(model, caches_b)):
            wf = model[l + 1]["P"].t["w_attn_pre"] if l + 1 < N else w_final
            B.beam_decode_stack(dims, dims.Fd, l, [_layer_struct(m, c)], wf, hb, xb, pt, seq,
                                rope, p, wsb)
        B.beam_check()
        assert torch.equal(ha, hb), f"step {step}: h differs"
        assert torch.equal(xa, xb), f"step {step}: x differs"
        for ca, cb in zip(caches_a, caches_b):
            assert torch.equal(ca.K, cb.K) and torch.equal(ca.V, cb.V)
        assert torch.isfinite(xa.view(torch.bfloat16).float()).all()


def test_stack_rejects_bad_layers():
    dims, model = _model("bf16")
    rope = rope_table(LMAX, dims.d, dims.theta)
    pt, st = dev(np.array([P0], np.int32)), dev(np.array([0], np.int32))
    h, x = torch.zeros((1, dims.D), **I16), torch.empty((1, dims.D), **I16)
    wsb = _stack_ws(dims)
    dense0 = _layer_struct(model[0], model[0]["cache"])
    with pytest.raises(B.BeamError) as e:        # a dense layer needs Fd
        B.beam_decode_stack(dims, 0, 0, [dense0], model[0]["P"].t["w_next_pre"], h, x, pt, st,
                            rope, P0, wsb)
    assert e.value.code == -2
    moe3 = _layer_struct(model[3], model[3]["cache"])
    moe3.w_r = None
    with pytest.raises(B.BeamError) as e:        # an MoE layer needs its router
        B.beam_decode_stack(dims, dims.Fd, 3, [moe3], model[3]["P"].t["w_next_pre"], h, x, pt, st,
                            rope, P0, wsb)
    assert e.value.code == -1
    with pytest.raises(B.BeamError) as e:        # workspace too small
        B.beam_decode_stack(dims, dims.Fd, 0, [dense0], model[0]["P"].t["w_next_pre"], h, x, pt,
                            st, rope, P0, wsb[:1024])
    assert e.value.code == -5
