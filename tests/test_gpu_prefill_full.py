"""Chunked prefill at full size, in the launch configuration the benchmark
times: 8 sequences x 2048 new tokens, each after 100,000 prior tokens of a bf16
cache (Lmax 102,400), through the NoPE MoE layer, the SWA MoE layer and the
dense layer 0 of the Beam shape (hidden 5120, 48/8 heads of 128, 256 experts).

The whole layer runs on the GPU through the C calls (many-token GEMMs, grouped
expert GEMMs, the flash attention kernel); the oracle then checks sampled
tokens stage by stage, each stage fed the GPU's upstream tensors, to the same
bar as the small-size stage tests. The oracle's attention reads the GPU-written
cache (prior positions drawn by the shared generator, the chunk's own keys
checked against the oracle's k/v write first)."""
import numpy as np
import pytest
import torch

import synth
from beamrun import Cache, Params, assert_rms_close, bits_f64, check_routing, run_layer
from oracle import layer as L
from oracle.numerics import bf16_bits_to_f64, round_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

# (sequence, index in its 2048-token chunk): first/last tokens of a chunk, the
# first sequence's start, interior tokens, the last sequence's end
SAMPLES = [(0, 0), (0, 1), (0, 1000), (0, 2047), (5, 7), (5, 2047), (7, 512), (7, 2046)]
MOE_SAMPLES = 4  # tokens whose routed experts are recomputed (8 expert fetches each)


class DeviceKV:
    """Oracle-side view of the GPU cache (bf16): keys(s, j, lo, hi) as float64,
    fetched per (sequence, kv head) on first use and kept for that sequence."""

    def __init__(self, cache: Cache, upto: int):
        self.c, self.upto = cache, upto
        self.s = None
        self.mem = {}

    def keys(self, s, j, lo, hi):
        if s != self.s:
            self.s, self.mem = s, {}
        if j not in self.mem:
            K = self.c.K[s, j, :self.upto].cpu().numpy().view(np.uint16)
            V = self.c.V[s, j, :, :self.upto].t().contiguous().cpu().numpy().view(np.uint16)
            self.mem[j] = (bf16_bits_to_f64(K), bf16_bits_to_f64(V))
        K, V = self.mem[j]
        return K[lo:hi + 1], V[lo:hi + 1]


def _run(kind):
    ex = synth.config(3).extra
    dims = synth.config(1).dims  # the Beam layer shape, as the benchmark's prefill leg
    S, C, prior, Lmax = ex["S"], ex["chunk"], ex["prior"], ex["Lmax"]
    layer = ex["layers"][kind]
    mode = "nope" if kind == "nope_moe" else "swa"  # layer 0 is a sliding-window layer
    ffn = "dense" if kind == "dense" else "moe"
    n = 2 * layer + 1
    torch.cuda.empty_cache()
    P = Params(dims, 0, layer, moe=(ffn == "moe"), dense=(ffn == "dense"), device_draw=True)
    Kp, Vp, ks, vs = synth.torch_kv_prior(dims, S, prior, "bf16", 0, layer)
    cache = Cache(dims, S, Lmax, "bf16", ks, vs)
    cache.fill_prior(Kp, Vp)
    del Kp, Vp
    pos = np.concatenate([np.arange(prior, prior + C) for _ in range(S)]).astype(np.int32)
    seq = np.repeat(np.arange(S), C).astype(np.int32)
    h = synth.torch_normal_bf16((S * C, dims.D), 1.0, 0, "prefill_h", kind)
    g = run_layer(dims, P, cache, h, pos, seq, mode, n, ffn=ffn)
    return dims, P, cache, g, pos, seq, mode, n, ffn, prior + C


def _check(dims, P, cache, g, pos, seq, mode, n, ffn, upto):
    eps = dims.eps
    ts = np.array([s * 2048 + c for s, c in SAMPLES])
    sel = lambda k: g[k][ts]  # noqa: E731
    # entry boundary, packed projection (whole rows of the sampled tokens)
    _, x_ref = L.boundary(None, sel("h_in"), None, P.np("w_attn_pre"), 0, eps)
    assert_rms_close(bits_f64(sel("x")), x_ref, "x")
    qkvg = L.qkvg_projection(sel("x"), P.np("w_qkvg"))
    nqkv = (dims.Hq + 2 * dims.Hkv) * dims.d
    assert_rms_close(bits_f64(sel("qkv")), qkvg[:, :nqkv], "qkv projection")
    if dims.G:
        assert_rms_close(bits_f64(sel("g")), qkvg[:, nqkv:nqkv + dims.G], "g")
    # per-head norm + position, fed the GPU's projection; the cache write
    q, k, v, _ = L.split_qkvg(dims, np.concatenate([bits_f64(sel("qkv")), qkvg[:, nqkv:]], 1))
    qn, kn = L.qk_norm_position(dims, q, k, pos[ts], mode, P.np("w_qnorm"), P.np("w_knorm"))
    assert_rms_close(bits_f64(sel("q")), round_bf16(qn), "q")
    for i, t in enumerate(ts):
        s, p = int(seq[t]), int(pos[t])
        kw = cache.K[s, :, p].cpu().numpy().view(np.uint16)
        vw = cache.V[s, :, :, p].cpu().numpy().view(np.uint16)
        assert_rms_close(bits_f64(kw), round_bf16(kn[i]), "k write")
        assert_rms_close(bits_f64(vw), v[i], "v write")
    # attention over the whole visible range (100K+ keys on NoPE layers), in
    # sequence order so each sequence's cache is fetched once
    o_ref = L.attention(dims, bits_f64(sel("q")), pos[ts], seq[ts], DeviceKV(cache, upto), mode,
                        P.np("sink") if "sink" in P.t else None)
    e_max = assert_rms_close(bits_f64(sel("o")), o_ref, "o")
    e_rms = float(np.sqrt(np.mean((bits_f64(sel("o")) - o_ref) ** 2)) / np.sqrt(np.mean(o_ref ** 2)))
    print(f"[prefill {mode}] attention output vs oracle: max|err| {e_max:.3e}, "
          f"rms(err) {e_rms:.3e} of rms(ref)", flush=True)
    z = L.output_gate(dims, bits_f64(sel("o")), bits_f64(sel("g")), P.np("b_gate"))
    assert_rms_close(bits_f64(sel("y")), L.o_proj(z, P.np("w_o")), "y")
    hm, _ = L.boundary(sel("y"), sel("h_in"), P.np("w_attn_post"), P.np("w_ffn_pre"), n, eps)
    assert_rms_close(bits_f64(sel("h_mid")), hm, "h_mid")
    _, x2 = L.boundary(None, sel("h_mid"), None, P.np("w_ffn_pre"), 0, eps)
    assert_rms_close(bits_f64(sel("x2")), x2, "x2")
    if ffn == "moe":
        check_routing(dims, sel("x2"), P, sel("idx"), sel("w"), sel("logits"), "router")
        m = ts[:MOE_SAMPLES]
        y2 = L.moe(dims, g["x2"][m], g["idx"][m], g["w"][m], P.expert)
        assert_rms_close(bits_f64(g["y2"][m]), y2, "y2")
        ts = m
    else:
        y2 = L.dense_ffn(sel("x2"), P.np("dense_w13"), P.np("dense_w2"), dims.Fd)
        assert_rms_close(bits_f64(sel("y2")), y2, "y2")
    ho, _ = L.boundary(g["y2"][ts], g["h_mid"][ts], P.np("w_ffn_post"), P.np("w_next_pre"),
                       n + 1, eps)
    assert_rms_close(bits_f64(g["h_out"][ts]), ho, "h_out")
    _, xn = L.boundary(None, g["h_out"][ts], None, P.np("w_next_pre"), 0, eps)
    assert_rms_close(bits_f64(g["x_next"][ts]), xn, "x_next")


@pytest.mark.parametrize("kind", ["nope_moe", "swa_moe", "dense"])
def test_full_size_prefill(kind):
    r = _run(kind)
    print(f"[prefill {kind}] GPU layer done", flush=True)
    _check(*r)
