"""Per-call parity of the HIP path against the oracle, each call fed the same
seeded inputs (GPU)."""
import numpy as np
import pytest
import torch

import moe_decoder_layer_amd as B
import synth
from beamrun import (Cache, Params, assert_rms_close, bits_f64, check_routing, code_pos, dev,
                     host_bits, rope_table, ws, ws_payload)
from oracle import layer as L
from oracle.numerics import e4m3_quantize, round_bf16

pytestmark = pytest.mark.gpu

CFG0 = synth.config(0).dims
BEAM = synth.config(1).dims
FLINT = synth.config(4).dims  # 256 experts, sigmoid top-6, no groups
I16 = dict(dtype=torch.int16, device="cuda")


def _dims(base, **kw):
    return synth.with_dims(synth.Config("", base), **kw).dims


# ------------------------------------------------------------------ boundary
@pytest.mark.parametrize("D,T", [(256, 1), (256, 37), (5120, 1), (5120, 600)])
@pytest.mark.parametrize("case", ["entry", "n5", "n1", "plain"])
def test_boundary(D, T, case):
    dims = _dims(CFG0, D=D)
    h = synth.make_h((T, D), 1, "bh", D, T)
    y = synth.make_h((T, D), 1, "by", D, T)
    wp = synth.uniform_bf16((D,), 0.5, 1.5, 1, "wp", D)
    wn = synth.uniform_bf16((D,), 0.5, 1.5, 1, "wn", D)
    hd, x = dev(h), torch.empty((T, D), **I16)
    if case == "entry":
        B.beam_boundary_norm_residual(dims, T, None, None, hd, dev(wn), x, 0)
        h_ref, x_ref = L.boundary(None, h, None, wn, 0, dims.eps)
    elif case == "plain":
        B.beam_boundary_norm_residual(dims, T, dev(y), None, hd, dev(wn), x, 0)
        h_ref, x_ref = L.boundary(y, h, None, wn, 0, dims.eps)
    else:
        n = 5 if case == "n5" else 1
        B.beam_boundary_norm_residual(dims, T, dev(y), dev(wp), hd, dev(wn), x, n)
        h_ref, x_ref = L.boundary(y, h, wp, wn, n, dims.eps)
    B.beam_check()
    hg, xg = bits_f64(host_bits(hd)), bits_f64(host_bits(x))
    assert_rms_close(hg, h_ref, "h")
    # the pre-norm is checked on the stored h it normalises
    _, x_of_h = L.boundary(None, host_bits(hd), None, wn, 0, dims.eps)
    assert_rms_close(xg, x_of_h, "x")
    assert np.mean(hg == h_ref) > 0.97 and np.mean(xg == x_of_h) > 0.97


# ------------------------------------------------------------------ q/k + cache write
@pytest.mark.parametrize("base,T,pos0", [(CFG0, 1, 64), (CFG0, 32, 64), (BEAM, 1, 3000),
                                         (BEAM, 3, 17), (BEAM, 40, 1000)])
@pytest.mark.parametrize("mode", ["swa", "nope"])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_qk_norm_kvwrite(base, T, pos0, mode, kv):
    dims = base
    Lmax = 4096 if dims.D > 1000 else 128
    P = Params(dims, 0, 3, moe=False)
    x = synth.make_h((T, dims.D), 2, "qx", T)
    pos = np.arange(pos0, pos0 + T, dtype=np.int32)
    seq = (np.arange(T) % 2).astype(np.int32)
    cache = Cache(dims, 2, Lmax, kv, 0.013, 0.021)
    q = torch.empty((T, dims.Hq, dims.d), **I16)
    g = torch.empty((T, dims.G), **I16)
    rope = rope_table(Lmax, dims.d, dims.theta) if mode == "swa" else None
    wsq = ws(dims, B.BEAM_OP_QKV, T)
    B.beam_qk_norm_rope_ssmax_kvwrite(
        dims, T, dev(x), P.t["w_qkvg"], P.t["w_qnorm"], P.t["w_knorm"], dev(pos), dev(seq),
        B.BEAM_SWA_ROPE if mode == "swa" else B.BEAM_NOPE_SSMAX, rope, q, g, cache.struct(), wsq)
    B.beam_check()
    qkvg = L.qkvg_projection(x, P.np("w_qkvg"))
    nqkv = (dims.Hq + 2 * dims.Hkv) * dims.d
    # the projection (first rounding point) against the oracle; the per-head
    # stage against the oracle fed the GPU's stored projection
    gq = ws_payload(wsq, T * nqkv * 2).view(torch.int16).view(T, nqkv)
    assert_rms_close(bits_f64(host_bits(gq)), qkvg[:, :nqkv], "qkv projection")
    qkv_gpu = np.concatenate([bits_f64(host_bits(gq)), qkvg[:, nqkv:]], axis=1)
    qr, kr, vr, gr = L.split_qkvg(dims, qkv_gpu)
    _, _, _, gr = L.split_qkvg(dims, qkvg)
    qn, kn = L.qk_norm_position(dims, qr, kr, pos, mode, P.np("w_qnorm"), P.np("w_knorm"))
    assert_rms_close(bits_f64(host_bits(q)), round_bf16(qn), "q")
    assert_rms_close(bits_f64(host_bits(g)), gr, "g")
    K = cache.K.cpu().numpy()
    V = cache.V.cpu().numpy()
    for t in range(T):
        s, p = seq[t], pos[t]
        kg, vg = K[s, :, p, :], V[s, :, :, p]
        if kv == "bf16":
            assert_rms_close(bits_f64(kg.view(np.uint16)), round_bf16(kn[t]), "k")
            assert_rms_close(bits_f64(vg.view(np.uint16)), vr[t], "v")
        else:
            for got, ref, sc in ((kg, kn[t], 0.013), (vg, vr[t], 0.021)):
                assert np.max(np.abs(code_pos(got) - code_pos(e4m3_quantize(ref, sc)))) <= 1
    # nothing outside the written slots changed
    mask = np.ones(K.shape[:3], bool)
    for t in range(T):
        mask[seq[t], :, pos[t]] = False
    fill = 0x7FC0 if kv == "bf16" else 0x7F
    assert np.all(K.view(np.uint16 if kv == "bf16" else np.uint8)[mask] == fill)


@pytest.mark.parametrize("case", ["tiny", "beam_near", "beam_mid", "beam_far", "beam_nogate",
                                  "flint_sink"])
@pytest.mark.parametrize("mode", ["swa", "nope"])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_attn_decode_fused(case, mode, kv):
    """One-token fused attention half against the separate calls: the q it
    reports and the cache bytes it writes equal those of the q/k call bit for
    bit, and its gated output matches the oracle's gate over the attention of
    those same inputs (the stage bar). Spans cover the one-pass workgroup
    (tiny), the merge by the last workgroup (beam_near, SWA at any position)
    and the merge kernel (beam_mid / beam_far NoPE: 12 / 47 chunks); the
    position sits on a tile edge in beam_far. beam_nogate: no output gate
    (z = o); flint_sink: the second model's shape with per-head sinks."""
    if case == "tiny":
        dims, Lmax, fill, p = CFG0, 192, 150, 100
    elif case == "beam_near":
        dims, Lmax, fill, p = BEAM, 4096, 3000, 1000
    elif case == "beam_mid":
        dims, Lmax, fill, p = BEAM, 4096, 3000, 2999
    elif case == "beam_far":
        dims, Lmax, fill, p = BEAM, 12096, 12032, 11968
    elif case == "beam_nogate":
        dims, Lmax, fill, p = _dims(BEAM, G=0), 4096, 3000, 2047
    else:
        dims, Lmax, fill, p = FLINT, 1024, 900, 700
    P = Params(dims, 0, 3, moe=False)
    x = dev(synth.make_h((1, dims.D), 2, "fx", case))
    pos, seq = np.array([p], np.int32), np.array([1], np.int32)
    Kp, Vp, ks, vs = synth.torch_kv_prior(dims, 2, fill, kv, 5, 9)
    c_ref = Cache(dims, 2, Lmax, kv, ks, vs)
    c_ref.fill_prior(Kp, Vp)
    c_fus = c_ref.clone()
    rope = rope_table(Lmax, dims.d, dims.theta) if mode == "swa" else None
    m = B.BEAM_SWA_ROPE if mode == "swa" else B.BEAM_NOPE_SSMAX
    sink = P.t.get("sink")
    # the separate calls
    q_ref = torch.empty((1, dims.Hq, dims.d), **I16)
    g_ref = torch.empty((1, max(dims.G, 1)), **I16)
    B.beam_qk_norm_rope_ssmax_kvwrite(dims, 1, x, P.t["w_qkvg"], P.t["w_qnorm"], P.t["w_knorm"],
                                      dev(pos), dev(seq), m, rope, q_ref,
                                      g_ref if dims.G else None, c_ref.struct(),
                                      ws(dims, B.BEAM_OP_QKV, 1))
    o_ref = torch.empty((1, dims.Hq, dims.d), **I16)
    attn = B.beam_attn_swa if mode == "swa" else B.beam_attn_nope_ssmax
    op = B.BEAM_OP_ATTN_SWA if mode == "swa" else B.BEAM_OP_ATTN_NOPE
    attn(dims, 1, q_ref, dev(pos), dev(seq), c_ref.struct(), sink, o_ref, p, ws(dims, op, 1, p + 1))
    # the fused call
    q_f = torch.empty((1, dims.Hq, dims.d), **I16)
    z_f = torch.full((1, dims.Hq * dims.d), 0x7FC0, **I16)
    B.beam_attn_decode_fused(dims, 1, x, P.t["w_qkvg"], P.t["w_qnorm"], P.t["w_knorm"],
                             dev(pos), dev(seq), m, rope, c_fus.struct(), sink, P.t.get("b_gate"),
                             q_f, z_f, p, ws(dims, B.BEAM_OP_ATTN_DECODE_FUSED, 1, p + 1))
    B.beam_check()
    assert torch.equal(q_f, q_ref), "fused q differs from the q/k call's"
    assert torch.equal(c_fus.K, c_ref.K) and torch.equal(c_fus.V, c_ref.V), "cache bytes differ"
    o_gpu = bits_f64(host_bits(o_ref))
    if dims.G:
        z_want = L.output_gate(dims, o_gpu, bits_f64(host_bits(g_ref)), P.np("b_gate"))
    else:
        z_want = o_gpu.reshape(1, -1)
    assert_rms_close(bits_f64(host_bits(z_f)), z_want, "z fused")
    # and the attention itself against the oracle on the same q and cache
    o_want = L.attention(dims, bits_f64(host_bits(q_ref)), pos, seq, c_ref.oracle(p + 1), mode,
                         P.np("sink") if sink is not None else None)
    assert_rms_close(o_gpu, o_want, "o")
    # o_proj on the gated output (no gate in the call): the weights-first GEMV
    y = torch.empty((1, dims.D), **I16)
    B.beam_out_gate(dims, 1, z_f, None, None, P.t["w_o"], y, ws(dims, B.BEAM_OP_OUT_GATE, 1))
    B.beam_check()
    assert_rms_close(bits_f64(host_bits(y)), L.o_proj(bits_f64(host_bits(z_f)), P.np("w_o")),
                     "y")


@pytest.mark.parametrize("base,T", [(BEAM, 1), (CFG0, 3), (BEAM, 40)])
def test_qk_slot_outside_cache_is_flagged(base, T):
    """A position at Lmax (or a slot index at S) skips that token's cache write
    and raises the device flag; the other tokens are written as usual."""
    dims = base
    Lmax = 128
    P = Params(dims, 0, 3, moe=False)
    x = synth.make_h((T, dims.D), 2, "qbad", T)
    cache = Cache(dims, 2, Lmax, "bf16", 1.0, 1.0)
    rope = rope_table(Lmax, dims.d, dims.theta)
    for pos, seq, msg in ((np.full(T, Lmax, np.int32), np.zeros(T, np.int32), "position"),
                          (np.arange(T, dtype=np.int32), np.full(T, 2, np.int32), "sequence")):
        q = torch.empty((T, dims.Hq, dims.d), **I16)
        g = torch.empty((T, dims.G), **I16)
        B.beam_qk_norm_rope_ssmax_kvwrite(
            dims, T, dev(x), P.t["w_qkvg"], P.t["w_qnorm"], P.t["w_knorm"], dev(pos), dev(seq),
            B.BEAM_SWA_ROPE, rope, q, g, cache.struct(), ws(dims, B.BEAM_OP_QKV, T))
        with pytest.raises(B.BeamError) as e:
            B.beam_check()
        assert e.value.code == -8 and msg in str(e.value)
        B.beam_check()                  # flag cleared
    assert np.all(cache.K.cpu().numpy().view(np.uint16) == 0x7FC0)
    assert np.all(cache.V.cpu().numpy().view(np.uint16) == 0x7FC0)


def _bits(v):
    from oracle.numerics import f64_to_bf16_bits
    return f64_to_bf16_bits(v)


# ------------------------------------------------------------------ attention
def _needle_cache(dims, Lmax, fill, kv, q, pos, seq, needles, seed):
    """Random N(0,1) prior over [0, fill) plus keys aligned with the token's
    first query head of each group at the needle positions (scores far above
    the rest, so a dropped or misplaced key changes the output)."""
    S = int(seq.max()) + 1
    Kp, Vp, ks, vs = synth.torch_kv_prior(dims, S, fill, kv, seed, 7)
    cache = Cache(dims, S, Lmax, kv, ks, vs)
    cache.fill_prior(Kp, Vp)
    grp = dims.Hq // dims.Hkv
    qf = bits_f64(host_bits(q))
    for t, p in enumerate(pos):
        for u in needles(int(p)):
            for j in range(dims.Hkv):
                qh = qf[t, j * grp]
                kvec = qh * (6.0 * np.sqrt(dims.d) / max(np.dot(qh, qh), 1e-6))
                if kv == "bf16":
                    cache.K[seq[t], j, u] = dev(_bits(kvec))
                else:
                    cache.K[seq[t], j, u] = torch.from_numpy(e4m3_quantize(kvec, ks)).cuda()
    return cache


@pytest.mark.parametrize("case", ["tiny", "tiny_few", "beam_multi", "beam_few", "beam_long",
                                  "beam_chunk", "beam_two_seq", "beam_mid", "beam_mid2",
                                  "group16_short", "group16"])
@pytest.mark.parametrize("mode", ["swa", "nope"])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_attention(case, mode, kv):
    """Few tokens (<= 4) take the split-K decode kernel: one chunk normalises
    in place (tiny_few, group16_short), up to 8 chunks merge in their last
    workgroup (SWA windows, beam_mid*), more in the merge kernel (beam_long,
    NoPE beam_few and group16); more tokens take the flash kernel. beam_two_seq:
    a flash-kernel block of 64 tokens holds the last 37 of one sequence and
    the first 27 of another, with different key ranges (one pass each, edge
    tiles at both ends of both ranges)."""
    seq = None
    if case == "beam_two_seq":
        dims, Lmax, fill = BEAM, 4096, 3063
        pos = np.concatenate([np.arange(1000, 1037), np.arange(3000, 3063)]).astype(np.int32)
        seq = np.repeat(np.array([0, 1], np.int32), [37, 63])
    elif case == "beam_mid":
        dims, Lmax, fill = BEAM, 4096, 3000
        pos = np.array([1500], np.int32)
    elif case == "beam_mid2":
        dims, Lmax, fill = BEAM, 4096, 3000
        pos = np.array([1200, 1900], np.int32)
    elif case == "group16_short":  # GQA group of 16, one chunk
        dims, Lmax, fill = _dims(BEAM, Hq=32, Hkv=2, G=0), 1024, 256
        pos = np.array([5, 200], np.int32)
    elif case == "group16":
        dims, Lmax, fill = _dims(BEAM, Hq=32, Hkv=2, G=0), 4096, 3000
        pos = np.array([64, 700, 2999], np.int32)
    elif case == "tiny":
        dims, Lmax, fill = CFG0, 192, 128
        pos = np.array([0, 15, 16, 63, 64, 100, 127], np.int32)
    elif case == "tiny_few":
        dims, Lmax, fill = CFG0, 192, 128
        pos = np.array([3, 64, 127], np.int32)
    elif case == "beam_few":
        dims, Lmax, fill = BEAM, 4096, 3000
        pos = np.array([700, 2999], np.int32)
    elif case == "beam_chunk":  # a prefill chunk: 70 consecutive tokens after 2900 prior
        dims, Lmax, fill = BEAM, 4096, 2970
        pos = np.arange(2900, 2970, dtype=np.int32)
    elif case == "beam_multi":
        dims, Lmax, fill = BEAM, 4096, 3000
        pos = np.array([0, 511, 512, 1000, 2047, 2999], np.int32)
    else:
        dims, Lmax, fill = BEAM, 100352, 100001
        pos = np.array([100000], np.int32)
    T = len(pos)
    if seq is None:
        seq = (np.arange(T) % 2).astype(np.int32) if case not in ("beam_long", "beam_chunk") \
            else np.zeros(T, np.int32)
    q = dev(synth.make_h((T, dims.Hq, dims.d), 3, "aq", case))
    W = dims.window

    def needles(p):
        c = {0, p, max(0, p - 1), max(0, p - W + 1), max(0, p - W), (p // 256) * 256,
             max(0, (p // 1024) * 1024 - 1)}
        return sorted(u for u in c if u <= p)

    cache = _needle_cache(dims, Lmax, fill, kv, q, pos, seq, needles, 4)
    o = torch.empty((T, dims.Hq, dims.d), **I16)
    sink = None
    mp = int(pos.max())
    fn = B.beam_attn_swa if mode == "swa" else B.beam_attn_nope_ssmax
    op = B.BEAM_OP_ATTN_SWA if mode == "swa" else B.BEAM_OP_ATTN_NOPE
    fn(dims, T, q, dev(pos), dev(seq), cache.struct(), sink, o, mp, ws(dims, op, T, mp + 1))
    B.beam_check()
    ref = L.attention(dims, bits_f64(host_bits(q)), pos, seq, cache.oracle(mp + 1), mode)
    assert_rms_close(bits_f64(host_bits(o)), ref, "o")


@pytest.mark.parametrize("mode", ["swa", "nope"])
def test_attention_sink(mode):
    dims = CFG0
    pos = np.array([5, 40, 99], np.int32)
    T = 3
    seq = np.zeros(T, np.int32)
    q = dev(synth.make_h((T, dims.Hq, dims.d), 3, "sq"))
    cache = _needle_cache(dims, 128, 128, "bf16", q, pos, seq, lambda p: [], 5)
    sink = torch.tensor([0.5, -1.0, 3.0, 8.0], dtype=torch.float32, device="cuda")
    o = torch.empty((T, dims.Hq, dims.d), **I16)
    fn = B.beam_attn_swa if mode == "swa" else B.beam_attn_nope_ssmax
    op = B.BEAM_OP_ATTN_SWA if mode == "swa" else B.BEAM_OP_ATTN_NOPE
    fn(dims, T, q, dev(pos), dev(seq), cache.struct(), sink, o, 99, ws(dims, op, T, 100))
    B.beam_check()
    ref = L.attention(dims, bits_f64(host_bits(q)), pos, seq, cache.oracle(100), mode,
                      sink=sink.cpu().numpy())
    assert_rms_close(bits_f64(host_bits(o)), ref, "o")


@pytest.mark.parametrize("mode", ["swa", "nope"])
def test_workspace_counters_reused(mode):
    """Split-K attention and the decode router elect a last workgroup with
    counters at the head of the workspace: repeated calls on one workspace
    give identical results and leave the counter block zeroed."""
    dims = BEAM
    pos = np.array([1499], np.int32)  # NoPE: 6 chunks merged by the last
    seq = np.zeros(1, np.int32)
    q = dev(synth.make_h((1, dims.Hq, dims.d), 7, "cq"))
    cache = _needle_cache(dims, 4096, 3000, "bf16", q, pos, seq, lambda p: [], 5)
    fn = B.beam_attn_swa if mode == "swa" else B.beam_attn_nope_ssmax
    op = B.BEAM_OP_ATTN_SWA if mode == "swa" else B.BEAM_OP_ATTN_NOPE
    w = ws(dims, op, 1, 3000)
    outs = []
    for _ in range(3):
        o = torch.empty((1, dims.Hq, dims.d), **I16)
        fn(dims, 1, q, dev(pos), dev(seq), cache.struct(), None, o, 1499, w)
        B.beam_check()
        assert int(w[:1024].count_nonzero()) == 0
        outs.append(o)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    ref = L.attention(dims, bits_f64(host_bits(q)), pos, seq, cache.oracle(1500), mode)
    assert_rms_close(bits_f64(host_bits(outs[0])), ref, "o")
    # the router shares the workspace (same stream): same counters, same result
    P = Params(dims, 0, 5, moe=False)
    x = dev(synth.make_h((1, dims.D), 6, "rx", 1))
    res = []
    for _ in range(3):
        idx = torch.empty((1, dims.topk), dtype=torch.int32, device="cuda")
        wt = torch.empty((1, dims.topk), dtype=torch.float32, device="cuda")
        B.beam_router_fp32_grouped_topk(dims, 1, x, P.t["w_r"], P.t["b_corr"], idx, wt, None, w)
        B.beam_check()
        assert int(w[:1024].count_nonzero()) == 0
        res.append((idx, wt))
    assert all(torch.equal(res[0][0], r[0]) and torch.equal(res[0][1], r[1]) for r in res)


@pytest.mark.parametrize("mode,max_pos,bad_pos", [("nope", 1499, 1699), ("nope", 2999, 3999),
                                                 ("swa", 100, 600)])
def test_attention_beyond_max_pos_is_flagged(mode, max_pos, bad_pos):
    """The split-K grid and its record stride are sized from the host's
    max_pos. A token past it is not attended: its output row is zero, the call
    reports the device flag, and the counter block is left zeroed, so the next
    call on the same workspace is correct. The cases take the three combine
    forms: merged by the last workgroup (NoPE, 6 chunks), by the merge kernel
    (NoPE, 12 chunks) and one pass with no records (SWA, one chunk). A valid
    token in the same call is unaffected."""
    dims = BEAM
    pos = np.array([min(max_pos, 1000), bad_pos], np.int32)
    seq = np.zeros(2, np.int32)
    q = dev(synth.make_h((2, dims.Hq, dims.d), 7, "mp", mode))
    cache = _needle_cache(dims, 4096, 4000, "bf16", q, pos, seq, lambda p: [0, p], 5)
    fn = B.beam_attn_swa if mode == "swa" else B.beam_attn_nope_ssmax
    op = B.BEAM_OP_ATTN_SWA if mode == "swa" else B.BEAM_OP_ATTN_NOPE
    w = ws(dims, op, 2, max_pos + 1)
    o = torch.full((2, dims.Hq, dims.d), 0x3F80, **I16)  # 1.0: a row left unwritten shows
    fn(dims, 2, q, dev(pos), dev(seq), cache.struct(), None, o, max_pos, w)
    with pytest.raises(B.BeamError) as e:
        B.beam_check()
    assert e.value.code == -8 and "max_pos" in str(e.value)
    assert int(w[:1024].count_nonzero()) == 0
    assert int(o[1].count_nonzero()) == 0
    qf = bits_f64(host_bits(q))
    ref = L.attention(dims, qf[:1], pos[:1], seq[:1], cache.oracle(max_pos + 1), mode)
    assert_rms_close(bits_f64(host_bits(o[:1])), ref, "o (valid token)")
    # the next call on the same workspace, at max_pos itself
    p2 = np.array([max_pos], np.int32)
    o2 = torch.empty((1, dims.Hq, dims.d), **I16)
    fn(dims, 1, q[1:2].contiguous(), dev(p2), dev(seq[:1]), cache.struct(), None, o2, max_pos, w)
    B.beam_check()
    assert int(w[:1024].count_nonzero()) == 0
    ref2 = L.attention(dims, qf[1:2], p2, seq[:1], cache.oracle(max_pos + 1), mode)
    assert_rms_close(bits_f64(host_bits(o2)), ref2, "o (next call)")


@pytest.mark.parametrize("mode", ["swa", "nope"])
def test_prefill_attention_flags(mode):
    """The many-token kernel on a bf16 cache at head dim 128 takes P.V on fp16
    operands. A cached value beyond fp16's range (7e4) is clamped to 65504 and
    the call reports the device flag; the output then equals the oracle's
    attention over the cache with that value clamped. The largest bf16 value
    below 65536 (65280) converts exactly and is not reported. A token at a
    negative position is reported and its output row is zero."""
    dims = BEAM
    T = 70
    pos = np.arange(2900, 2970, dtype=np.int32)
    seq = np.zeros(T, np.int32)
    q = dev(synth.make_h((T, dims.Hq, dims.d), 3, "vclamp", mode))
    cache = _needle_cache(dims, 4096, 2970, "bf16", q, pos, seq, lambda p: [], 5)
    oc = cache.oracle(2970)
    u = 2950 if mode == "nope" else 2960   # inside every later token's window
    cache.V[0, 3, 17, u] = dev(_bits(np.array([7.0e4])))[0]
    oc.V[0, 3, u, 17] = 65504.0
    fn = B.beam_attn_swa if mode == "swa" else B.beam_attn_nope_ssmax
    op = B.BEAM_OP_ATTN_SWA if mode == "swa" else B.BEAM_OP_ATTN_NOPE
    o = torch.empty((T, dims.Hq, dims.d), **I16)
    fn(dims, T, q, dev(pos), dev(seq), cache.struct(), None, o, 2969, ws(dims, op, T, 2970))
    with pytest.raises(B.BeamError) as e:
        B.beam_check()
    assert e.value.code == -8 and "fp16" in str(e.value)
    ref = L.attention(dims, bits_f64(host_bits(q)), pos, seq, oc, mode)
    assert_rms_close(bits_f64(host_bits(o)), ref, "o (value clamped)")
    # a negative position: reported, row zero, the other tokens unchanged; the
    # value at 65280 is in fp16's range (no range report)
    pos2 = pos.copy()
    pos2[5] = -1
    cache.V[0, 3, 17, u] = dev(_bits(np.array([65280.0])))[0]
    oc.V[0, 3, u, 17] = 65280.0
    o2 = torch.empty((T, dims.Hq, dims.d), **I16)
    fn(dims, T, q, dev(pos2), dev(seq), cache.struct(), None, o2, 2969, ws(dims, op, T, 2970))
    with pytest.raises(B.BeamError) as e:
        B.beam_check()
    assert e.value.code == -8 and "outside the cache" in str(e.value)
    assert "fp16" not in str(e.value)
    assert int(o2[5].count_nonzero()) == 0
    keep = np.arange(T) != 5
    ref2 = L.attention(dims, bits_f64(host_bits(q))[keep], pos[keep], seq[keep], oc, mode)
    assert_rms_close(bits_f64(host_bits(o2))[keep], ref2, "o (other tokens)")


# ------------------------------------------------------------------ gate + o_proj
@pytest.mark.parametrize("base,T", [(CFG0, 1), (CFG0, 9), (BEAM, 1), (BEAM, 2),
                                    ("beam_no_gate", 1), ("beam_no_gate", 3)])
def test_out_gate(base, T):
    """Output gate + o_proj against the oracle; the Beam shape without an
    output gate runs o_proj on the attention output as it is."""
    dims = _dims(BEAM, G=0) if base == "beam_no_gate" else base
    P = Params(dims, 0, 4, moe=False)
    o = synth.make_h((T, dims.Hq * dims.d), 5, "go", T)
    y = torch.empty((T, dims.D), **I16)
    if dims.G:
        g = synth.make_h((T, dims.G), 5, "gg", T)
        B.beam_out_gate(dims, T, dev(o), dev(g), P.t["b_gate"], P.t["w_o"], y,
                        ws(dims, B.BEAM_OP_OUT_GATE, T))
        z = L.output_gate(dims, bits_f64(o).reshape(T, dims.Hq, dims.d), bits_f64(g),
                          P.np("b_gate"))
    else:
        B.beam_out_gate(dims, T, dev(o), None, None, P.t["w_o"], y,
                        ws(dims, B.BEAM_OP_OUT_GATE, T))
        z = bits_f64(o)
    B.beam_check()
    assert_rms_close(bits_f64(host_bits(y)), L.o_proj(z, P.np("w_o")), "y")


# ------------------------------------------------------------------ router
@pytest.mark.parametrize("base,T", [(CFG0, 1), (CFG0, 70), (BEAM, 1), (BEAM, 4), (BEAM, 300),
                                    (FLINT, 1), (FLINT, 3), (FLINT, 128), ("beam_all_groups", 1),
                                    ("beam_all_groups", 40)])
def test_router(base, T):
    """Grouped selection (top groups, then top experts) and, with no groups or
    every group kept (the second model's layer; the Beam shape with all 8
    groups kept), the plain top-k path, each against the oracle."""
    if base == "beam_all_groups":
        base = _dims(BEAM, topk_group=8)
    dims = base
    P = Params(dims, 0, 5, moe=False)
    x = synth.make_h((T, dims.D), 6, "rx", T)
    idx = torch.empty((T, dims.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, dims.topk), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, dims.E), dtype=torch.float32, device="cuda")
    B.beam_router_fp32_grouped_topk(dims, T, dev(x), P.t["w_r"], P.t["b_corr"], idx, w, lg,
                                    ws(dims, B.BEAM_OP_ROUTER, T))
    B.beam_check()
    check_routing(dims, x, P, idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy(), "router")
    # without logits output (workspace path) the selection is identical
    idx2 = torch.empty_like(idx)
    w2 = torch.empty_like(w)
    B.beam_router_fp32_grouped_topk(dims, T, dev(x), P.t["w_r"], P.t["b_corr"], idx2, w2, None,
                                    ws(dims, B.BEAM_OP_ROUTER, T))
    assert torch.equal(idx, idx2) and torch.equal(w, w2)


def _tie_sets(dims, P):
    """Make the router rows and biases of each set of five consecutive experts
    inside a group (the last set of a group may be shorter) repeat the set's
    first; returns each expert's set leader."""
    gs = dims.E // max(dims.n_group, 1)
    e = np.arange(dims.E)
    lead = e - e % gs + 5 * ((e % gs) // 5)
    for k in ("w_r", "b_corr"):
        if P.t.get(k) is not None:
            a = np.array(P.np(k)[lead], copy=True)
            P._np[k], P.t[k] = a, dev(a)
    return lead


@pytest.mark.parametrize("base,T", [(BEAM, 1), (BEAM, 300), ("beam_all_groups", 1),
                                    ("beam_all_groups", 40), (FLINT, 1), (FLINT, 128)])
def test_router_exact_ties(base, T):
    """Exact ties: inside each expert group, experts come in sets of five
    consecutive indices whose router rows and biases repeat the set's first
    (the last set of a group may be shorter), so a set's logits and biased
    scores are equal bit for bit. Five does not divide top-k (8 or 6), so sets
    straddle the selection boundary; the selection must then take a set's
    lowest indices. Checked on the GPU's own logits (rounding cannot undo an
    exact tie) and against the oracle."""
    if base == "beam_all_groups":
        base = _dims(BEAM, topk_group=8)
    dims = base
    P = Params(dims, 0, 5, moe=False)
    lead = _tie_sets(dims, P)
    x = synth.make_h((T, dims.D), 6, "rt", T)
    idx = torch.empty((T, dims.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, dims.topk), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, dims.E), dtype=torch.float32, device="cuda")
    B.beam_router_fp32_grouped_topk(dims, T, dev(x), P.t["w_r"], P.t["b_corr"], idx, w, lg,
                                    ws(dims, B.BEAM_OP_ROUTER, T))
    B.beam_check()
    lgh, idh = lg.cpu().numpy(), idx.cpu().numpy()
    assert np.array_equal(lgh.view(np.uint32), lgh[:, lead].view(np.uint32))
    split = 0
    for t in range(T):
        sel = set(idh[t].tolist())
        assert len(sel) == dims.topk
        for j in sel:
            assert all(i in sel for i in range(lead[j], j)), \
                f"token {t}: expert {j} taken before a lower index of its tie set"
        split += any(j + 1 < dims.E and lead[j + 1] == lead[j] and j + 1 not in sel
                     for j in sel)
    assert split > 0, "no tie set straddles the selection boundary"
    check_routing(dims, x, P, idh, w.cpu().numpy(), lgh, "router ties")


@pytest.mark.parametrize("base,T,ties", [(CFG0, 1, False), (BEAM, 1, False), (BEAM, 3, False),
                                         (BEAM, 1, True), ("beam_all_groups", 1, True)])
def test_boundary_router_fused_equals_calls(base, T, ties):
    """The fused boundary + router call gives the two calls' results bit for
    bit (T = 1 runs as one kernel), also when repeated on one workspace, and
    with exact ties in the router scores (sets of five equal experts)."""
    dims = _dims(BEAM, topk_group=8) if base == "beam_all_groups" else base
    P = Params(dims, 0, 5, moe=False)
    lead = _tie_sets(dims, P) if ties else None
    y = dev(synth.make_h((T, dims.D), 8, "fy", T))
    h0 = synth.make_h((T, dims.D), 9, "fh", T)
    n = 21

    def outs():
        return (torch.empty((T, dims.topk), dtype=torch.int32, device="cuda"),
                torch.empty((T, dims.topk), dtype=torch.float32, device="cuda"),
                torch.empty((T, dims.E), dtype=torch.float32, device="cuda"),
                torch.empty((T, dims.D), **I16))
    h1 = dev(h0)
    i1, w1, l1, x1 = outs()
    B.beam_boundary_norm_residual(dims, T, y, P.t["w_attn_post"], h1, P.t["w_ffn_pre"], x1, n)
    B.beam_router_fp32_grouped_topk(dims, T, x1, P.t["w_r"], P.t["b_corr"], i1, w1, l1,
                                    ws(dims, B.BEAM_OP_ROUTER, T))
    wsf = ws(dims, B.BEAM_OP_ROUTER, T)
    for _ in range(2):
        h2 = dev(h0)
        i2, w2, l2, x2 = outs()
        B.beam_boundary_router_fp32_grouped_topk(dims, T, y, P.t["w_attn_post"], h2,
                                                 P.t["w_ffn_pre"], x2, n, P.t["w_r"],
                                                 P.t["b_corr"], i2, w2, l2, wsf)
        B.beam_check()
        for a, b, name in ((h1, h2, "h"), (x1, x2, "x"), (i1, i2, "idx"), (w1, w2, "w"),
                           (l1, l2, "logits")):
            assert torch.equal(a, b), name
        assert int(wsf[:1024].count_nonzero()) == 0
        if ties:  # a tie set's lowest indices are the ones taken
            for row in i2.cpu().numpy():
                sel = set(row.tolist())
                assert all(i in sel for j in sel for i in range(lead[j], j)), row


# ------------------------------------------------------------------ experts
_BEAM_P = {}


def _beam_params():
    if "p" not in _BEAM_P:
        _BEAM_P["p"] = Params(BEAM, 0, 10, moe=True, device_draw=True)
    return _BEAM_P["p"]


@pytest.mark.parametrize("base,T", [(CFG0, 1), (CFG0, 5), (BEAM, 1), (BEAM, 2)])
def test_moe(base, T):
    dims = base
    P = Params(dims, 0, 6) if dims is CFG0 else _beam_params()
    x = synth.make_h((T, dims.D), 7, "mx", T)
    g = np.random.default_rng(8)
    idx = np.stack([g.choice(dims.E, dims.topk, replace=False) for _ in range(T)]).astype(np.int32)
    w = g.uniform(0.05, 0.6, (T, dims.topk)).astype(np.float32)
    y = torch.empty((T, dims.D), **I16)
    B.beam_moe_swiglu_combine(dims, T, dev(x), dev(idx), dev(w), P.t["w13"], P.t["w2"], None, None,
                              y, ws(dims, B.BEAM_OP_MOE, T))
    B.beam_check()
    ref = L.moe(dims, x, idx, w, P.expert)
    assert_rms_close(bits_f64(host_bits(y)), ref, "y2")


@pytest.mark.parametrize("T,bad", [(3, False), (40, False), (300, False), (40, True),
                                   (300, True)])
def test_moe_shared_expert(T, bad):
    """Shared expert beside the routed ones. T = 3 takes the one-token
    kernels; T = 40 (200 routed + shared pairs) the grouped GEMM's 32-row
    tiles; T = 300 (1,200 pairs, more than 16 per expert segment) its
    256-row tiles walked expert by expert, with the shared expert's weights
    taken from its own buffer for the last segment. bad: one routed id per
    row of a few rows is out of range; it is reported and left out, and the
    shared expert's row still lands in the combine."""
    dims = _dims(CFG0, shared=True, topk=3, n_group=1, topk_group=1)
    P = Params(dims, 0, 6)
    x = synth.make_h((T, dims.D), 7, "msx", T)
    g = np.random.default_rng(12)
    idx = np.stack([g.choice(dims.E, 3, replace=False) for _ in range(T)]).astype(np.int32)
    w = g.uniform(0.05, 0.6, (T, 3)).astype(np.float32)
    rows = [1, T // 2, T - 1]
    if bad:
        for r, v in zip(rows, (dims.E, -1, dims.E + 7)):
            idx[r, r % 3] = v
    y = torch.empty((T, dims.D), **I16)
    B.beam_moe_swiglu_combine(dims, T, dev(x), dev(idx), dev(w), P.t["w13"], P.t["w2"],
                              P.t["shared_w13"], P.t["shared_w2"], y, ws(dims, B.BEAM_OP_MOE, T))
    if bad:
        with pytest.raises(B.BeamError) as e:
            B.beam_check()
        assert e.value.code == -8
        for r in rows:  # any valid id not already in the row, at weight 0
            k = r % 3
            idx[r, k] = next(i for i in range(dims.E) if i not in idx[r])
            w[r, k] = 0.0
    B.beam_check()
    ref = L.moe(dims, x, idx, w, P.expert, shared=(P.np("shared_w13"), P.np("shared_w2")))
    assert_rms_close(bits_f64(host_bits(y)), ref, "y2")


@pytest.mark.parametrize("D", [64, 128, 192, 320])
def test_moe_sparse_tiles_short_k(D):
    """Many tokens with a few rows per expert (T = 40, 160 pairs over 16
    experts: 32-row tiles). The gate/up product stages its K slabs of 64
    through a ring of four; D = 64, 128, 192 and 320 give 1, 2, 3 and 5 slabs,
    so the ring's prologue, its waits near the end of K and its wrap-around
    all run."""
    dims = _dims(CFG0, D=D)
    T = 40
    P = Params(dims, 0, 6)
    x = synth.make_h((T, D), 7, "mshort", D)
    g = np.random.default_rng(D)
    idx = np.stack([g.choice(dims.E, dims.topk, replace=False) for _ in range(T)]).astype(np.int32)
    w = g.uniform(0.05, 0.6, (T, dims.topk)).astype(np.float32)
    y = torch.empty((T, D), **I16)
    B.beam_moe_swiglu_combine(dims, T, dev(x), dev(idx), dev(w), P.t["w13"], P.t["w2"], None, None,
                              y, ws(dims, B.BEAM_OP_MOE, T))
    B.beam_check()
    ref = L.moe(dims, x, idx, w, P.expert)
    assert_rms_close(bits_f64(host_bits(y)), ref, "y2")


@pytest.mark.parametrize("T", [256, 512, 513])
def test_moe_routing_pair_counts(T):
    """The routing permutation at the one-workgroup kernel's edges: 1,024 and
    2,048 (token, slot) pairs (one and two full batches of its ranking) and
    2,052 (past its limit: the chunked three-kernel path)."""
    dims = CFG0
    P = Params(dims, 0, 6)
    x = synth.make_h((T, dims.D), 7, "mroute", T)
    g = np.random.default_rng(T)
    idx = np.stack([g.choice(dims.E, dims.topk, replace=False) for _ in range(T)]).astype(np.int32)
    w = g.uniform(0.05, 0.6, (T, dims.topk)).astype(np.float32)
    y = torch.empty((T, dims.D), **I16)
    B.beam_moe_swiglu_combine(dims, T, dev(x), dev(idx), dev(w), P.t["w13"], P.t["w2"], None, None,
                              y, ws(dims, B.BEAM_OP_MOE, T))
    B.beam_check()
    ref = L.moe(dims, x, idx, w, P.expert)
    assert_rms_close(bits_f64(host_bits(y)), ref, "y2")


def test_moe_bad_expert_id_is_flagged():
    """An id outside [0, E) is skipped by the kernels' own check and reported."""
    dims = CFG0
    P = Params(dims, 0, 6)
    x = synth.make_h((1, dims.D), 7, "bad")
    idx = np.array([[1, 2, dims.E, 3]], np.int32)
    w = np.full((1, 4), 0.5, np.float32)
    y = torch.empty((1, dims.D), **I16)
    B.beam_moe_swiglu_combine(dims, 1, dev(x), dev(idx), dev(w), P.t["w13"], P.t["w2"], None, None,
                              y, ws(dims, B.BEAM_OP_MOE, 1))
    with pytest.raises(B.BeamError) as e:
        B.beam_check()
    assert e.value.code == -8
    B.beam_check()                      # flag cleared
    ref = L.moe(dims, x, np.array([[1, 2, 3]]), w[:, :3], P.expert)
    assert_rms_close(bits_f64(host_bits(y)), ref, "y2 without the bad slot")


@pytest.mark.parametrize("base,T", [(CFG0, 1), (CFG0, 6), (BEAM, 1)])
def test_dense(base, T):
    dims = base
    layer = 0
    if dims is CFG0:
        w13, w2 = synth.make_dense(dims, 0, layer)
        w13d, w2d = dev(w13), dev(w2)
    else:
        w13d = synth.torch_normal_bf16((2 * dims.Fd, dims.D), 0.02, 0, layer, "dense_w13")
        w2d = synth.torch_normal_bf16((dims.D, dims.Fd), 0.02, 0, layer, "dense_w2")
        w13, w2 = host_bits(w13d), host_bits(w2d)
    x = synth.make_h((T, dims.D), 9, "dx", T)
    y = torch.empty((T, dims.D), **I16)
    dd = _dims(dims, F=dims.Fd)
    B.beam_dense_swiglu(T, dims.D, dims.Fd, dev(x), w13d, w2d, y, ws(dd, B.BEAM_OP_DENSE, T))
    B.beam_check()
    assert_rms_close(bits_f64(host_bits(y)), L.dense_ffn(x, w13, w2, dims.Fd), "y2")


# ------------------------------------------------------------------ matrix-core paths at Beam shapes
@pytest.mark.parametrize("T", [300])
def test_qkv_gemm_beam(T):
    """Packed projection on the MFMA GEMM (ragged 256-row tiles) + epilogue."""
    test_qk_norm_kvwrite(BEAM, T, 17, "nope", "bf16")


def test_out_gate_gemm_beam():
    test_out_gate(BEAM, 300)


def test_moe_bad_expert_id_many_tokens():
    """Many tokens (routing permutation + grouped GEMMs): ids outside [0, E)
    are left out of the permutation, skipped by the combine and reported; the
    other pairs match the oracle with the rejected slots at weight 0."""
    dims = CFG0
    P = Params(dims, 0, 6)
    T = 40
    x = synth.make_h((T, dims.D), 7, "badm", T)
    g = np.random.default_rng(11)
    idx = np.stack([g.choice(dims.E, dims.topk, replace=False) for _ in range(T)]).astype(np.int32)
    w = g.uniform(0.05, 0.6, (T, dims.topk)).astype(np.float32)
    bad = [(7, 2, dims.E), (30, 0, -1), (39, 3, dims.E + 100)]
    for t, k, v in bad:
        idx[t, k] = v
    y = torch.empty((T, dims.D), **I16)
    B.beam_moe_swiglu_combine(dims, T, dev(x), dev(idx), dev(w), P.t["w13"], P.t["w2"], None, None,
                              y, ws(dims, B.BEAM_OP_MOE, T))
    with pytest.raises(B.BeamError) as e:
        B.beam_check()
    assert e.value.code == -8
    idx_ok, w_ok = idx.copy(), w.copy()
    for t, k, _ in bad:  # any valid id not already in the row, at weight 0
        idx_ok[t, k] = next(i for i in range(dims.E) if i not in idx[t])
        w_ok[t, k] = 0.0
    assert_rms_close(bits_f64(host_bits(y)), L.moe(dims, x, idx_ok, w_ok, P.expert), "y2")


def test_dense_gemm_beam():
    test_dense(BEAM, 300)


def test_moe_grouped_gemm_beam():
    """Grouped expert GEMMs: 300 tokens all routed to the same 8 experts, so each
    expert segment has 300 rows (one full and one ragged 256-row tile), plus
    a second run spread over 24 experts (single ragged tiles)."""
    dims = BEAM
    P = _beam_params()
    T = 300
    x = synth.make_h((T, dims.D), 7, "mgx")
    g = np.random.default_rng(9)
    for pool in (np.array([3, 17, 40, 99, 128, 200, 201, 255]), g.choice(256, 24, replace=False)):
        idx = np.stack([g.choice(pool, dims.topk, replace=False) for _ in range(T)]).astype(np.int32)
        w = g.uniform(0.05, 0.6, (T, dims.topk)).astype(np.float32)
        y = torch.empty((T, dims.D), **I16)
        B.beam_moe_swiglu_combine(dims, T, dev(x), dev(idx), dev(w), P.t["w13"], P.t["w2"], None,
                                  None, y, ws(dims, B.BEAM_OP_MOE, T))
        B.beam_check()
        assert_rms_close(bits_f64(host_bits(y)), L.moe(dims, x, idx, w, P.expert), "y2")
