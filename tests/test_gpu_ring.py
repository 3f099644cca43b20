"""Ring caches for the sliding-window layers ("Reflection Beam 1.0 on vLLM",
Attention section: those layers attend to their last 512 positions only). A
cache of Lmax slots per sequence that accepts positions up to npos > Lmax
keeps position p in slot p mod Lmax. The kernels are the linear-cache kernels
with that slot map, so every call on a ring gives the bit-identical result of
the same call on a linear cache that holds the same keys; one case per test
is also checked against the oracle (GPU)."""
import numpy as np
import pytest
import torch

import moe_decoder_layer_amd as B
import synth
from beamrun import Cache, Params, assert_rms_close, bits_f64, dev, host_bits, rope_table, ws
from oracle import layer as L

pytestmark = pytest.mark.gpu

BEAM = synth.config(1).dims  # window 512
I16 = dict(dtype=torch.int16, device="cuda")
NPOS = 1 << 20


class Ring(Cache):
    """Device cache of `slots` slots per sequence accepting positions below npos."""

    def __init__(self, dims, S, slots, npos, kv, k_scale=1.0, v_scale=1.0):
        super().__init__(dims, S, slots, kv, k_scale, v_scale)
        self.npos = npos

    def struct(self):
        return B.kv_struct(self.K, self.V,
                           B.BEAM_KV_BF16 if self.kv == "bf16" else B.BEAM_KV_FP8_E4M3,
                           self.k_scale, self.v_scale, self.S, self.Lmax, self.npos)


def _ring_of(lin: Cache, slots: int, upto: list[int]) -> Ring:
    """The ring state after sequence s wrote positions [0, upto[s]) in order:
    positions [upto[s] - slots, upto[s]) of the linear cache at slot p mod slots
    (slots never written keep the NaN fill)."""
    r = Ring(lin.dims, lin.S, slots, NPOS, lin.kv, lin.k_scale, lin.v_scale)
    for s, u in enumerate(upto):
        ps = torch.arange(max(0, u - slots), u, device="cuda")
        r.K[s, :, ps % slots] = lin.K[s, :, ps]
        r.V[s, :, :, ps % slots] = lin.V[s, :, :, ps]
    return r


def _case(case):
    """(S, ring slots, pos, seq) of an attention case."""
    g = np.random.default_rng(3)
    if case == "decode":        # one token past several wraps
        return 2, 512, [5000], [1]
    if case == "decode_576":    # a ring one tile larger than the window
        return 2, 576, [4999], [0]
    if case == "few":           # split-K, three sequences (a 512-slot ring holds the
        return 3, 512, [4000, 4711, 3333], [0, 1, 2]  # window of one token per sequence)
    if case == "batch":         # a batch of decode steps, one per sequence
        S = 48
        return S, 512, list(g.integers(600, 5000, S)), list(range(S))
    if case == "chunk":         # a prefill chunk (flash kernel): ring >= window + 69
        return 1, 640, list(range(4900, 4970)), [0] * 70
    # two chunks of 100 tokens in one call (flash kernel)
    return 2, 640, list(range(3000, 3100)) + list(range(4500, 4600)), [0] * 100 + [1] * 100


@pytest.mark.parametrize("case", ["decode", "decode_576", "few", "batch", "chunk", "two_chunks"])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_ring_attention_equals_linear(case, kv):
    dims = BEAM
    S, slots, pos, seq = _case(case)
    pos, seq = np.array(pos, np.int32), np.array(seq, np.int32)
    T = len(pos)
    upto = [int(pos[seq == s].max()) + 1 if np.any(seq == s) else 0 for s in range(S)]
    ctx = max(upto)
    Kp, Vp, ks, vs = synth.torch_kv_prior(dims, S, ctx, kv, 21, 4)
    lin = Cache(dims, S, (ctx + 63) // 64 * 64, kv, ks, vs)
    lin.fill_prior(Kp, Vp)
    del Kp, Vp
    ring = _ring_of(lin, slots, upto)
    q = dev(synth.make_h((T, dims.Hq, dims.d), 3, "ring_q", case))
    mp = int(pos.max())
    outs = []
    for c in (lin, ring):
        o = torch.empty((T, dims.Hq, dims.d), **I16)
        B.beam_attn_swa(dims, T, q, dev(pos), dev(seq), c.struct(), None, o, mp,
                        ws(dims, B.BEAM_OP_ATTN_SWA, T, mp + 1))
        B.beam_check()
        outs.append(o)
    assert torch.equal(outs[0], outs[1]), "ring and linear caches give different outputs"
    if kv == "bf16" and case in ("decode", "batch", "two_chunks"):
        want = L.attention(dims, bits_f64(host_bits(q)), pos, seq, lin.oracle(ctx), "swa")
        assert_rms_close(bits_f64(host_bits(outs[1])), want, "o (ring)")


@pytest.mark.parametrize("T", [1, 3, 40, 300])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_ring_qk_write(T, kv):
    """The q/k call writes position p's key and value to slot p mod Lmax (RoPE
    at the absolute position) with the bytes the linear cache gets at p."""
    dims = BEAM
    S, slots, npos = 2, 512, 8192
    if T == 1:
        pos, seq = [5000], [1]
    elif T == 3:
        pos, seq = [5000, 5001, 700], [0, 0, 1]
    elif T == 40:
        pos, seq = list(range(4000, 4040)), [0] * 40
    else:
        pos, seq = list(range(7000, 7300)), [1] * 300
    pos, seq = np.array(pos, np.int32), np.array(seq, np.int32)
    P = Params(dims, 0, 3, moe=False)
    x = dev(synth.make_h((T, dims.D), 2, "ring_x", T))
    rope = rope_table(npos, dims.d, dims.theta)
    ks, vs = (1.0, 1.0) if kv == "bf16" else (0.02, 0.02)
    lin = Cache(dims, S, npos, kv, ks, vs)
    ring = Ring(dims, S, slots, npos, kv, ks, vs)
    qs = []
    for c in (lin, ring):
        q = torch.empty((T, dims.Hq, dims.d), **I16)
        g = torch.empty((T, dims.G), **I16)
        B.beam_qk_norm_rope_ssmax_kvwrite(dims, T, x, P.t["w_qkvg"], P.t["w_qnorm"],
                                          P.t["w_knorm"], dev(pos), dev(seq), B.BEAM_SWA_ROPE,
                                          rope, q, g, c.struct(), ws(dims, B.BEAM_OP_QKV, T))
        B.beam_check()
        qs.append(q)
    assert torch.equal(qs[0], qs[1])
    pt, st = torch.from_numpy(pos).long().cuda(), torch.from_numpy(seq).long().cuda()
    assert torch.equal(ring.K[st, :, pt % slots], lin.K[st, :, pt])
    assert torch.equal(ring.V[st, :, :, pt % slots], lin.V[st, :, :, pt])
    # a NoPE layer's full-context cache cannot be a ring
    with pytest.raises(B.BeamError) as e:
        B.beam_qk_norm_rope_ssmax_kvwrite(dims, T, x, P.t["w_qkvg"], P.t["w_qnorm"],
                                          P.t["w_knorm"], dev(pos), dev(seq), B.BEAM_NOPE_SSMAX,
                                          None, qs[1], None, ring.struct(),
                                          ws(dims, B.BEAM_OP_QKV, T))
    assert e.value.code == -3


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_ring_decode_steps_across_the_wrap(kv):
    """Consecutive fused decode steps (the q/k epilogue writes the new key and
    value into the ring, then attends) at positions 1000 to 1159, across the
    wrap at position 1024 (slot 0): each step's output and the written slot
    equal those of the same steps on a linear cache."""
    dims = BEAM
    S, slots, p0, n = 2, 512, 1000, 160
    P = Params(dims, 0, 5, moe=False)
    Kp, Vp, ks, vs = synth.torch_kv_prior(dims, S, p0, kv, 8, 2)
    lin = Cache(dims, S, 2048, kv, ks, vs)
    lin.fill_prior(Kp, Vp)
    ring = _ring_of(lin, slots, [p0, p0])
    rope = rope_table(2048, dims.d, dims.theta)
    ring.npos = 2048
    seq = np.array([1], np.int32)
    w = ws(dims, B.BEAM_OP_ATTN_DECODE_FUSED, 1, p0 + n)
    for k in range(n):
        p = p0 + k
        pos = np.array([p], np.int32)
        x = dev(synth.make_h((1, dims.D), 6, "ring_step", k))
        zs = []
        for c in (lin, ring):
            z = torch.empty((1, dims.Hq * dims.d), **I16)
            B.beam_attn_decode_fused(dims, 1, x, P.t["w_qkvg"], P.t["w_qnorm"], P.t["w_knorm"],
                                     dev(pos), dev(seq), B.BEAM_SWA_ROPE, rope, c.struct(), None,
                                     P.t["b_gate"], None, z, p, w)
            zs.append(z)
        B.beam_check()
        assert torch.equal(zs[0], zs[1]), f"step at position {p}: outputs differ"
        assert torch.equal(ring.K[1, :, p % slots], lin.K[1, :, p])
        assert torch.equal(ring.V[1, :, :, p % slots], lin.V[1, :, :, p])


def test_ring_rejections():
    """A NoPE (full-context) attention call rejects a ring; so does a window
    larger than the ring, and a position at or beyond npos is not attended
    (zero output, device flag)."""
    dims = BEAM
    ring = Ring(dims, 1, 512, 4096, "bf16")
    q = torch.zeros((1, dims.Hq, dims.d), **I16)
    o = torch.empty((1, dims.Hq, dims.d), **I16)
    pos, seq = dev(np.array([100], np.int32)), dev(np.array([0], np.int32))
    with pytest.raises(B.BeamError) as e:
        B.beam_attn_nope_ssmax(dims, 1, q, pos, seq, ring.struct(), None, o, 100,
                               ws(dims, B.BEAM_OP_ATTN_NOPE, 1, 101))
    assert e.value.code == -3
    small = Ring(dims, 1, 448, 4096, "bf16")
    with pytest.raises(B.BeamError) as e:
        B.beam_attn_swa(dims, 1, q, pos, seq, small.struct(), None, o, 100,
                        ws(dims, B.BEAM_OP_ATTN_SWA, 1, 101))
    assert e.value.code == -2
    with pytest.raises(B.BeamError) as e:
        B.beam_attn_swa(dims, 1, q, pos, seq, ring.struct(), None, o, 4096,
                        ws(dims, B.BEAM_OP_ATTN_SWA, 1, 4097))
    assert e.value.code == -2
    far = dev(np.array([4096], np.int32))
    o.fill_(7)
    B.beam_attn_swa(dims, 1, q, far, seq, ring.struct(), None, o, 4095,
                    ws(dims, B.BEAM_OP_ATTN_SWA, 1, 4096))
    with pytest.raises(B.BeamError) as e:
        B.beam_check()
    assert e.value.code == -8
    assert int(o.count_nonzero()) == 0
