"""The allocation-free NoPE attention entry point against the workspace one
(GPU). Same kernels, so the outputs must be bit-identical; both are also held
to the stage bar against the oracle. Two calls in a row, the second smaller,
so the shared static array's leftover records and counters are exercised."""
import numpy as np
import pytest
import torch

import moe_decoder_layer_amd as B
import synth
from beamrun import Cache, assert_rms_close, bits_f64, dev, host_bits, ws
from oracle import layer as L

pytestmark = pytest.mark.gpu

BEAM = synth.config(1).dims
I16 = dict(dtype=torch.int16, device="cuda")


def _case(kv, T, fill, Lmax, seed):
    S = 2
    Kp, Vp, ks, vs = synth.torch_kv_prior(BEAM, S, fill, kv, seed, 31)
    cache = Cache(BEAM, S, Lmax, kv, ks, vs)
    cache.fill_prior(Kp, Vp)
    q = dev(synth.make_h((T, BEAM.Hq, BEAM.d), seed, "static_q", T))
    return cache, q


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_static_attention_matches_workspace_call(kv):
    cache, q = _case(kv, 3, 9000, 9024, 3)
    # (tokens, positions, sequences): the second call is smaller (fewer tokens,
    # shorter spans, fewer chunks) than the first
    calls = [(np.array([8999, 4100, 6500], np.int32), np.array([0, 1, 0], np.int32)),
             (np.array([700], np.int32), np.array([1], np.int32))]
    for pos, seq in calls:
        T = len(pos)
        qq = q[:T].contiguous()
        mp = int(pos.max())
        o_ws = torch.empty((T, BEAM.Hq, BEAM.d), **I16)
        o_st = torch.full((T, BEAM.Hq, BEAM.d), 0x7FC0, **I16)
        B.beam_attn_nope_ssmax(BEAM, T, qq, dev(pos), dev(seq), cache.struct(), None, o_ws, mp,
                               ws(BEAM, B.BEAM_OP_ATTN_NOPE, T, mp + 1))
        B.beam_attn_nope_ssmax_static(BEAM, T, qq, dev(pos), dev(seq), cache.struct(), None,
                                      o_st, mp)
        B.beam_check()
        assert torch.equal(o_ws, o_st), f"static call differs from the workspace call at T={T}"
        ref = L.attention(BEAM, bits_f64(host_bits(qq)), pos, seq, cache.oracle(mp + 1), "nope")
        assert_rms_close(bits_f64(host_bits(o_st)), ref, "o static")


def test_static_attention_rejects_oversized_call():
    T = 128
    cache, q = _case("bf16", T, 64, 131072, 4)
    pos = np.full(T, 99999, np.int32)
    seq = np.zeros(T, np.int32)
    o = torch.empty((T, BEAM.Hq, BEAM.d), **I16)
    with pytest.raises(B.BeamError) as e:
        B.beam_attn_nope_ssmax_static(BEAM, T, q, dev(pos), dev(seq), cache.struct(), None, o,
                                      99999)
    assert e.value.code == -5 and "static" in str(e.value)
