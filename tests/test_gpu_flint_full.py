"""The second model's layer at full size, in the launch configuration the
benchmark times: 128 sequences, one new token each at position 8,192 of a
bf16 cache (Lmax 8,448), 256 experts (sigmoid top-6 without groups) plus a
shared expert, per-head sinks, pre-norm plain residual, SWA (513 keys) and
NoPE. The layer runs on the GPU through the C calls; the oracle then checks
sampled tokens stage by stage, each stage fed the GPU's upstream tensors, to
the same bar as the small-size tests, reading the GPU-written cache."""
import numpy as np
import pytest
import torch

import synth
from beamrun import Cache, Params, assert_rms_close, bits_f64, check_routing, run_layer
from oracle import layer as L
from oracle.numerics import round_bf16
from test_gpu_prefill_full import DeviceKV

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

SAMPLES = [0, 1, 37, 64, 101, 127]   # token = sequence index
LAYER = 3


@pytest.mark.parametrize("mode", ["swa", "nope"])
def test_full_size_batch_decode(mode):
    cfg = synth.config(4)
    dims, ex = cfg.dims, cfg.extra
    S, ctx, Lmax = ex["B"], ex["ctx"], ex["Lmax"]
    torch.cuda.empty_cache()
    P = Params(dims, 0, LAYER, moe=True, device_draw=True)
    Kp, Vp, ks, vs = synth.torch_kv_prior(dims, S, ctx, "bf16", 0, LAYER)
    cache = Cache(dims, S, Lmax, "bf16", ks, vs)
    cache.fill_prior(Kp, Vp)
    del Kp, Vp
    pos = np.full(S, ctx, np.int32)
    seq = np.arange(S, dtype=np.int32)
    h = synth.torch_normal_bf16((S, dims.D), 1.0, 0, "flint_full_h", mode)
    g = run_layer(dims, P, cache, h, pos, seq, mode, 0, sandwich=False)
    print(f"[flint full {mode}] GPU layer done", flush=True)

    eps, ts = dims.eps, np.array(SAMPLES)
    sel = lambda k: g[k][ts]  # noqa: E731
    _, x_ref = L.boundary(None, sel("h_in"), None, P.np("w_attn_pre"), 0, eps)
    assert_rms_close(bits_f64(sel("x")), x_ref, "x")
    qkvg = L.qkvg_projection(sel("x"), P.np("w_qkvg"))
    nqkv = (dims.Hq + 2 * dims.Hkv) * dims.d
    assert_rms_close(bits_f64(sel("qkv")), qkvg[:, :nqkv], "qkv projection")
    q, k, v, _ = L.split_qkvg(dims, bits_f64(sel("qkv")))
    qn, kn = L.qk_norm_position(dims, q, k, pos[ts], mode, P.np("w_qnorm"), P.np("w_knorm"))
    assert_rms_close(bits_f64(sel("q")), round_bf16(qn), "q")
    for i, t in enumerate(ts):
        kw = cache.K[seq[t], :, pos[t]].cpu().numpy().view(np.uint16)
        vw = cache.V[seq[t], :, :, pos[t]].cpu().numpy().view(np.uint16)
        assert_rms_close(bits_f64(kw), round_bf16(kn[i]), "k write")
        assert_rms_close(bits_f64(vw), v[i], "v write")
    o_ref = L.attention(dims, bits_f64(sel("q")), pos[ts], seq[ts], DeviceKV(cache, ctx + 1),
                        mode, P.np("sink"))
    assert_rms_close(bits_f64(sel("o")), o_ref, "o")
    z = bits_f64(sel("o")).reshape(len(ts), -1)
    assert_rms_close(bits_f64(sel("y")), L.o_proj(z, P.np("w_o")), "y")
    hm, _ = L.boundary(sel("y"), sel("h_in"), None, P.np("w_ffn_pre"), 0, eps)
    assert_rms_close(bits_f64(sel("h_mid")), hm, "h_mid")
    _, x2 = L.boundary(None, sel("h_mid"), None, P.np("w_ffn_pre"), 0, eps)
    assert_rms_close(bits_f64(sel("x2")), x2, "x2")
    check_routing(dims, sel("x2"), P, sel("idx"), sel("w"), sel("logits"), "router")
    shared = (P.np("shared_w13"), P.np("shared_w2"))
    y2 = L.moe(dims, sel("x2"), sel("idx"), sel("w"), P.expert, shared)
    assert_rms_close(bits_f64(sel("y2")), y2, "y2")
    ho, _ = L.boundary(sel("y2"), sel("h_mid"), None, P.np("w_next_pre"), 0, eps)
    assert_rms_close(bits_f64(sel("h_out")), ho, "h_out")
    _, xn = L.boundary(None, sel("h_out"), None, P.np("w_next_pre"), 0, eps)
    assert_rms_close(bits_f64(sel("x_next")), xn, "x_next")
