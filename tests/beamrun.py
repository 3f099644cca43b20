"""Test-side harness: seeded inputs on the device, the layer driven through the
C ABI (via the binding), and the oracle fed the same bytes.

Test infrastructure (imports the oracle). Not collected by pytest (no test_
prefix)."""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import moe_decoder_layer_amd as B
import synth
from oracle import layer as L
from oracle.numerics import bf16_bits_to_f64, e4m3_decode

BF16_NAN = 0x7FC0
FP8_NAN = 0x7F


# ----------------------------------------------------------------- conversions
def dev(a, device="cuda"):
    """numpy -> device tensor; uint16 (bf16 bits) travel as int16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def host_bits(t) -> np.ndarray:
    """device int16 tensor -> numpy uint16 bf16 bits."""
    return t.detach().cpu().numpy().view(np.uint16)


def host_f64(t) -> np.ndarray:
    return bf16_bits_to_f64(host_bits(t))


def bits_f64(a) -> np.ndarray:
    return bf16_bits_to_f64(a)


# ----------------------------------------------------------------- comparisons
def rms(a) -> float:
    a = np.asarray(a, np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def bf16_ulp(ref) -> np.ndarray:
    """Spacing of bf16 values at |ref| (8 significant bits)."""
    a = np.abs(np.asarray(ref, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(np.maximum(e, -126) - 7), 0.0)


# Every parity comparison of a session: (test, quantity, max|err|/rms(ref),
# rms(err)/rms(ref), elements). The test session prints the worst per
# quantity at its end; BEAM_PARITY_LOG names a file that gets every record.
PARITY: list[dict] = []


def _record(name, **kv):
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    rec = dict(test=test, name=name, **kv)
    PARITY.append(rec)
    path = os.environ.get("BEAM_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def assert_rms_close(got, ref, name="", frac=1e-2, ulps=1):
    """Parity bar for bf16 tensors: every element within
    max(frac * rms(ref), ulps bf16 ulps at the larger of the two elements'
    magnitudes), and the RMS of the error within frac * rms(ref).

    The ulp allowance exists because the tensors are bf16: where the GPU's fp32
    value and the oracle's float64 value straddle a rounding boundary the two
    roundings differ by one ulp, and above 2.56 * rms one bf16 ulp is larger
    than 1e-2 * rms. Stage comparisons feed the oracle the GPU's stored
    upstream tensors, so one rounding point separates them (ulps=1); whole-layer
    comparisons chain two (h_mid then h_out, ulps=2).
    Returns max|got - ref| / rms(ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite GPU values"
    if got.size == 0:
        return 0.0
    err = np.abs(got - ref)
    r = rms(ref)
    tol = frac * r
    # bf16 spacing at the larger of the two magnitudes: across a binade edge
    # (ref just below a power of two, got just above) the spacing doubles
    ulp = bf16_ulp(np.maximum(np.abs(ref), np.abs(got)))
    bad = err > np.maximum(tol, ulps * ulp * 1.0000001)
    assert not np.any(bad), (f"{name}: {int(bad.sum())} of {err.size} elements beyond "
                             f"max({frac}*rms, {ulps} ulp); worst |err| {err.max():.3e}, "
                             f"rms {r:.3e}")
    assert rms(err) <= tol, f"{name}: rms(err) {rms(err):.3e} > {frac} * rms {r:.3e}"
    e_max = float(err.max() / max(r, 1e-30))
    _record(name.split(" (")[0], max_rel=e_max, rms_rel=float(rms(err) / max(r, 1e-30)),
            n=int(err.size))
    return e_max


def code_pos(c):
    """Signed position of an e4m3 code on the number line (adjacent values differ by 1)."""
    c = np.asarray(c, np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


# ----------------------------------------------------------------- caches
class Cache:
    """Physical cache on the device (K [S][Hkv][Lmax][d], V^T [S][Hkv][d][Lmax]),
    unused slots filled with NaN patterns, plus its logical view for the oracle."""

    def __init__(self, dims, S, Lmax, kv="bf16", k_scale=1.0, v_scale=1.0):
        self.dims, self.S, self.Lmax, self.kv = dims, S, Lmax, kv
        self.k_scale, self.v_scale = k_scale, v_scale
        if kv == "bf16":
            self.K = torch.full((S, dims.Hkv, Lmax, dims.d), BF16_NAN, dtype=torch.int16,
                                device="cuda")
            self.V = torch.full((S, dims.Hkv, dims.d, Lmax), BF16_NAN, dtype=torch.int16,
                                device="cuda")
        else:
            self.K = torch.full((S, dims.Hkv, Lmax, dims.d), FP8_NAN, dtype=torch.uint8,
                                device="cuda")
            self.V = torch.full((S, dims.Hkv, dims.d, Lmax), FP8_NAN, dtype=torch.uint8,
                                device="cuda")

    def fill_prior(self, K, V):
        """K, V logical [S][Hkv][ctx][d] device tensors (int16 bits or uint8 codes)."""
        ctx = K.shape[2]
        self.K[:, :, :ctx] = K
        self.V[:, :, :, :ctx] = V.transpose(2, 3)

    def struct(self):
        return B.kv_struct(self.K, self.V,
                           B.BEAM_KV_BF16 if self.kv == "bf16" else B.BEAM_KV_FP8_E4M3,
                           self.k_scale, self.v_scale, self.S, self.Lmax)

    def oracle(self, upto: int | None = None) -> L.KVCache:
        """Logical oracle cache holding positions [0, upto) (the rest zero)."""
        upto = self.Lmax if upto is None else upto
        K = self.K[:, :, :upto].cpu().numpy()
        V = self.V[:, :, :, :upto].transpose(2, 3).contiguous().cpu().numpy()
        c = L.KVCache.empty(self.S, self.dims.Hkv, upto, self.dims.d, self.kv,
                            self.k_scale, self.v_scale)
        if self.kv == "bf16":
            c.K[:] = bf16_bits_to_f64(K.view(np.uint16))
            c.V[:] = bf16_bits_to_f64(V.view(np.uint16))
        else:
            c.K[:] = K
            c.V[:] = V
        return c

    def clone(self):
        c = Cache.__new__(Cache)
        c.__dict__.update(self.__dict__)
        c.K, c.V = self.K.clone(), self.V.clone()
        return c


def rope_table(Lmax, d, theta):
    t = np.zeros((Lmax, d), np.float32)
    B.beam_rope_table(t, Lmax, d, theta)
    return torch.from_numpy(t).cuda()


# ----------------------------------------------------------------- params
SMALL = ("w_attn_pre", "w_attn_post", "w_ffn_pre", "w_ffn_post", "w_next_pre", "w_qnorm",
         "w_knorm", "w_qkvg", "b_gate", "w_o", "w_r", "b_corr", "sink", "shared_w13",
         "shared_w2")


class Params:
    """Layer weights on the device. Small configs upload synth's numpy draws;
    full-size configs draw on the device (experts one by one)."""

    def __init__(self, dims, seed, layer, moe=True, dense=False, device_draw=False):
        self.dims = dims
        self.t = {}
        self._np = {}
        if not device_draw:
            p = synth.make_params(dims, seed, layer, experts=moe, dense=dense)
            self._np = p
            for k, v in p.items():
                self.t[k] = dev(v)
            return
        p = synth.make_params(dims, seed, layer, experts=False, projections=False)
        self._np.update(p)
        for k, v in p.items():
            self.t[k] = dev(v)
        self.t["w_qkvg"] = synth.torch_normal_bf16((dims.qkvg_rows, dims.D), 0.02, seed, layer,
                                                   "w_qkvg")
        self.t["w_o"] = synth.torch_normal_bf16((dims.D, dims.Hq * dims.d), 0.02, seed, layer,
                                                "w_o")
        if moe:
            w13 = torch.empty((dims.E, 2 * dims.F, dims.D), dtype=torch.int16, device="cuda")
            w2 = torch.empty((dims.E, dims.D, dims.F), dtype=torch.int16, device="cuda")
            for e in range(dims.E):
                synth.torch_normal_bf16((2 * dims.F, dims.D), 0.02, seed, layer, "w13", e,
                                        out=w13[e])
                synth.torch_normal_bf16((dims.D, dims.F), 0.02, seed, layer, "w2", e, out=w2[e])
            self.t["w13"], self.t["w2"] = w13, w2
            if dims.shared:
                self.t["shared_w13"] = synth.torch_normal_bf16((2 * dims.F, dims.D), 0.02, seed,
                                                               layer, "w13", "shared")
                self.t["shared_w2"] = synth.torch_normal_bf16((dims.D, dims.F), 0.02, seed,
                                                              layer, "w2", "shared")
        if dense:
            self.t["dense_w13"] = synth.torch_normal_bf16((2 * dims.Fd, dims.D), 0.02, seed,
                                                          layer, "dense_w13")
            self.t["dense_w2"] = synth.torch_normal_bf16((dims.D, dims.Fd), 0.02, seed, layer,
                                                         "dense_w2")

    def np(self, name):
        if name not in self._np:
            t = self.t[name]
            self._np[name] = host_bits(t) if t.dtype == torch.int16 else t.cpu().numpy()
        return self._np[name]

    def expert(self, e):
        return host_bits(self.t["w13"][e]), host_bits(self.t["w2"][e])

    def oracle_dict(self, experts=False):
        d = {k: self.np(k) for k in SMALL if k in self.t}
        if experts:
            d["w13"], d["w2"] = self.np("w13"), self.np("w2")
        if "dense_w13" in self.t:
            d["dense_w13"], d["dense_w2"] = self.np("dense_w13"), self.np("dense_w2")
        return d


# ----------------------------------------------------------------- GPU layer
CTL_BYTES = 1024  # counter block at the head of every workspace


def ws_payload(w, nbytes):
    """The first nbytes of a workspace's data area (after the counter block)."""
    return w[CTL_BYTES:CTL_BYTES + nbytes]


def ws(dims, op, T, ctx=0):
    n = B.beam_workspace_size(dims, op, T, ctx)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")  # counter block zeroed


def run_layer(dims, P: Params, cache: Cache, h_bits, pos, seq, mode: str, n: int,
              ffn="moe", rope=None, keep=True, sandwich=True, fused=False) -> dict:
    """One layer through the C ABI. Returns host copies of every intermediate.
    sandwich False: the pre-norm, plain-residual layer form (no post-norms).
    fused: the attention half through beam_attn_decode_fused (one token), then
    o_proj alone on its gated output; "z" replaces "o" in the result."""
    T = len(pos)
    D = dims.D
    t = P.t
    out = {}
    h = dev(h_bits) if isinstance(h_bits, np.ndarray) else h_bits.clone()
    pos_t = torch.as_tensor(np.asarray(pos, np.int32)).cuda()
    seq_t = torch.as_tensor(np.asarray(seq, np.int32)).cuda()
    I16 = dict(dtype=torch.int16, device="cuda")
    x = torch.empty((T, D), **I16)
    B.beam_boundary_norm_residual(dims, T, None, None, h, t["w_attn_pre"], x, 0)
    q = torch.empty((T, dims.Hq, dims.d), **I16)
    g = torch.empty((T, max(dims.G, 1)), **I16)
    kvs = cache.struct()
    m = B.BEAM_SWA_ROPE if mode == "swa" else B.BEAM_NOPE_SSMAX
    if rope is None and mode == "swa":
        rope = rope_table(cache.Lmax, dims.d, dims.theta)
    nqkv = (dims.Hq + 2 * dims.Hkv) * dims.d
    max_pos = int(np.max(pos))
    y = torch.empty((T, D), **I16)
    if fused:
        wsf = ws(dims, B.BEAM_OP_ATTN_DECODE_FUSED, T, max_pos + 1)
        z = torch.empty((T, dims.Hq * dims.d), **I16)
        B.beam_attn_decode_fused(dims, T, x, t["w_qkvg"], t["w_qnorm"], t["w_knorm"], pos_t,
                                 seq_t, m, rope if mode == "swa" else None, kvs, t.get("sink"),
                                 t.get("b_gate"), q, z, max_pos, wsf)
        out["qkv"] = host_bits(ws_payload(wsf, T * nqkv * 2).view(torch.int16).view(T, nqkv))
        goff = -(-T * nqkv * 2 // 256) * 256  # the gate follows the 256-aligned q|k|v rows
        if dims.G:
            g = ws_payload(wsf, goff + T * dims.G * 2)[goff:].view(torch.int16).view(T, dims.G)
        B.beam_out_gate(dims, T, z, None, None, t["w_o"], y, ws(dims, B.BEAM_OP_OUT_GATE, T))
        out["z"], o = host_bits(z), None
    else:
        wsq = ws(dims, B.BEAM_OP_QKV, T)
        B.beam_qk_norm_rope_ssmax_kvwrite(dims, T, x, t["w_qkvg"], t["w_qnorm"], t["w_knorm"],
                                          pos_t, seq_t, m, rope if mode == "swa" else None, q,
                                          g if dims.G else None, kvs, wsq)
        out["qkv"] = host_bits(ws_payload(wsq, T * nqkv * 2).view(torch.int16).view(T, nqkv))
        o = torch.empty((T, dims.Hq, dims.d), **I16)
        attn = B.beam_attn_swa if mode == "swa" else B.beam_attn_nope_ssmax
        op = B.BEAM_OP_ATTN_SWA if mode == "swa" else B.BEAM_OP_ATTN_NOPE
        attn(dims, T, q, pos_t, seq_t, kvs, t.get("sink"), o, max_pos,
             ws(dims, op, T, max_pos + 1))
        B.beam_out_gate(dims, T, o, g if dims.G else None, t.get("b_gate"), t["w_o"], y,
                        ws(dims, B.BEAM_OP_OUT_GATE, T))
    h_in = h.clone()
    x2 = torch.empty((T, D), **I16)
    if sandwich:
        B.beam_boundary_norm_residual(dims, T, y, t["w_attn_post"], h, t["w_ffn_pre"], x2, n)
    else:
        B.beam_boundary_norm_residual(dims, T, y, None, h, t["w_ffn_pre"], x2, 0)
    h_mid = h.clone()
    y2 = torch.empty((T, D), **I16)
    if ffn == "moe":
        idx = torch.empty((T, dims.topk), dtype=torch.int32, device="cuda")
        w = torch.empty((T, dims.topk), dtype=torch.float32, device="cuda")
        logits = torch.empty((T, dims.E), dtype=torch.float32, device="cuda")
        B.beam_router_fp32_grouped_topk(dims, T, x2, t["w_r"], t["b_corr"], idx, w, logits,
                                        ws(dims, B.BEAM_OP_ROUTER, T))
        B.beam_moe_swiglu_combine(dims, T, x2, idx, w, t["w13"], t["w2"], t.get("shared_w13"),
                                  t.get("shared_w2"), y2, ws(dims, B.BEAM_OP_MOE, T))
        out.update(idx=idx.cpu().numpy(), w=w.cpu().numpy(), logits=logits.cpu().numpy())
    else:
        dd = synth.with_dims(synth.Config("", dims), F=dims.Fd).dims
        B.beam_dense_swiglu(T, D, dims.Fd, x2, t["dense_w13"], t["dense_w2"], y2,
                            ws(dd, B.BEAM_OP_DENSE, T))
    xn = torch.empty((T, D), **I16)
    if sandwich:
        B.beam_boundary_norm_residual(dims, T, y2, t["w_ffn_post"], h, t["w_next_pre"], xn, n + 1)
    else:
        B.beam_boundary_norm_residual(dims, T, y2, None, h, t["w_next_pre"], xn, 0)
    B.beam_check()
    out.update(x=host_bits(x), q=host_bits(q), g=host_bits(g),
               o=host_bits(o) if o is not None else None, y=host_bits(y),
               h_in=host_bits(h_in), h_mid=host_bits(h_mid), x2=host_bits(x2), y2=host_bits(y2),
               h_out=host_bits(h), x_next=host_bits(xn))
    return out


def near_tie(margins_group, margins_expert, thr=1e-4):
    return (np.asarray(margins_group) <= thr) | (np.asarray(margins_expert) <= thr)


def router_logit_bound(x_f64, w_r):
    """Per-logit bar for the fp32 router: 1e-5 of the logit itself plus one
    binary32 unit (2^-24) of sum_i |x_i| |w_i|, the scale of the rounding
    error an fp32 accumulation of that dot product can carry (a logit that
    cancels to near zero keeps the rounding error of the terms it summed)."""
    absdot = np.abs(np.asarray(x_f64, np.float64)) @ np.abs(np.asarray(w_r, np.float64)).T
    return absdot * 2.0 ** -24


def check_routing(dims, x2_bits, P: Params, gpu_idx, gpu_w, gpu_logits, name=""):
    """Router parity: each logit within 1e-5 * |ref| + 2^-24 * sum_i |x_i||w_i|
    (router_logit_bound); idx sets exact where both selection margins exceed
    1e-4, else tie-consistent; weights from the GPU's own selection within
    1e-5 relative. Returns the near-tie mask."""
    x = bits_f64(x2_bits)
    r = L.router(dims, x, P.np("w_r"), P.np("b_corr"))
    ref = r["logits"].astype(np.float64)
    err = np.abs(np.asarray(gpu_logits, np.float64) - ref)
    bound = 1e-5 * np.abs(ref) + router_logit_bound(x, P.np("w_r"))
    ratio = err / bound
    _record(f"{name or 'router'} logits |err|/bound", max_rel=float(ratio.max()),
            rms_rel=float(err.max() / max(rms(ref), 1e-30)), n=int(err.size))
    assert ratio.max() <= 1.0, (f"{name}: router logit |err| {err.ravel()[ratio.argmax()]:.2e} "
                                f"beyond its bound {bound.ravel()[ratio.argmax()]:.2e}")
    tie = near_tie(r["group_margin"], r["expert_margin"])
    for t in range(len(gpu_idx)):
        gs = set(gpu_idx[t].tolist())
        if not tie[t]:
            assert gs == set(r["idx"][t].tolist()), f"{name}: token {t} idx {gs} vs {r['idx'][t]}"
        else:  # any selection whose scores tie the oracle's to within the margin
            sb = r["sb"][t].astype(np.float64)
            assert abs(sb[list(gs)].sum() - sb[r["idx"][t]].sum()) <= dims.topk * 2e-4
        s = r["s"][t][gpu_idx[t]].astype(np.float64)
        np.testing.assert_allclose(gpu_w[t], dims.route_scale * s / s.sum(), rtol=1e-5)
    return tie
