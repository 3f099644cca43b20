"""The Beam sparse decoder layer, computed plainly on the CPU in float64
(test infrastructure only; see oracle/__init__.py).

Source: the "Reflection Beam 1.0 on vLLM" page (and its Arabic and Chinese
renderings). Section names below are that page's:
  [Attn]   "Attention: sliding-window layers and NoPE full-attention layers"
  [MoE]    "MoE and residual stream: FP32 router, sandwich norm, depth-scaled residual"
  [Opt]    "Agent-driven optimisation makes batch-1 decode 2.71x faster" (7-item list)
and, for the second model, the "vLLM Day-0 support: Recursive's Flint" page,
section "Flint model architecture" [Flint].

Precision. Arithmetic is float64. The pages fix two precisions, and both are
kept: the router is FP32 end to end ([MoE]: weights, accumulation, logits),
so its logits are float64 sums rounded once to binary32 and every routing
decision is taken on binary32 values; and the fused kernels keep FP32 maths
with bf16 rounding at the reference's rounding points ([Opt], item 1), which
are marked below with round_bf16 (`bf`). The pages do not list those points;
the reading used is: every tensor that lands in memory between steps is bf16,
the cache is bf16 or fp8, the router's tensors are fp32, and every sum,
norm statistic, softmax and the expert combine is wide.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .numerics import (bf16_bits_to_f64, e4m3_decode, e4m3_quantize, round_bf16,
                       round_f32)

F64 = np.float64
bf = round_bf16


def as_f64(bits_or_values) -> np.ndarray:
    """bf16 bit patterns (uint16) decode to float64; float arrays pass through."""
    a = np.asarray(bits_or_values)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(F64)


# ----------------------------------------------------------------------------
# RMSNorm and the depth-scaled residual  [MoE]
# ----------------------------------------------------------------------------

def rms_norm(v, w, eps: float) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) * w over the last axis (gain w, no 1+w form)."""
    v = np.asarray(v, dtype=F64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * np.asarray(w, F64)


def scaled_residual(h, x, n: int) -> np.ndarray:
    """The n-th residual add: h <- sqrt((n-1)/n) h + x / sqrt(n)  [MoE].

    n = 0 selects the plain add h + x of a pre-norm layer [Flint]."""
    h = np.asarray(h, F64)
    x = np.asarray(x, F64)
    if n == 0:
        return h + x
    return math.sqrt((n - 1) / n) * h + x / math.sqrt(n)


def boundary(y, h, w_post, w_pre, n: int, eps: float):
    """Sublayer boundary: post-norm of the sublayer output y, the n-th scaled
    residual add into h, and the next sublayer's pre-norm  ([MoE] sandwich norm;
    [Opt] item 1 fuses exactly these three).

    y None: only the pre-norm x = rms(h) (the layer entry).
    w_post None: y is added without a post-norm (pre-norm layers, [Flint]).
    Returns (h_new, x), both bf16-exact float64.
    """
    h = as_f64(h)
    if y is not None:
        a = as_f64(y) if w_post is None else bf(rms_norm(as_f64(y), as_f64(w_post), eps))
        h = bf(scaled_residual(h, a, n))
    return h, bf(rms_norm(h, as_f64(w_pre), eps))


# ----------------------------------------------------------------------------
# Attention half  [Attn], [Opt] items 2, 5, 6
# ----------------------------------------------------------------------------

def qkvg_projection(x, w_qkvg) -> np.ndarray:
    """One GEMM over the packed [q | k | v | gate] weight ([Opt] item 5)."""
    return bf(as_f64(x) @ as_f64(w_qkvg).T)


def split_qkvg(dims, qkvg):
    T = qkvg.shape[0]
    a = dims.Hq * dims.d
    b = a + dims.Hkv * dims.d
    c = b + dims.Hkv * dims.d
    q = qkvg[:, :a].reshape(T, dims.Hq, dims.d)
    k = qkvg[:, a:b].reshape(T, dims.Hkv, dims.d)
    v = qkvg[:, b:c].reshape(T, dims.Hkv, dims.d)
    g = qkvg[:, c:c + dims.G]
    return q, k, v, g


def rope(v, pos, theta: float) -> np.ndarray:
    """Rotary position embedding, rotate-half pairing (i, i + d/2), frequency
    theta^(-2i/d), applied at integer position pos. v: [..., d]."""
    d = v.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=F64)
    ang = float(pos) * theta ** (-2.0 * i / d)
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def ssmax_factor(p) -> F64:
    """SSMax query scale (1 + p/2048)^0.1 with p the 1-based position  [Attn]."""
    return (1.0 + np.asarray(p, F64) / 2048.0) ** 0.1


def qk_norm_position(dims, q, k, pos, mode: str, w_qnorm, w_knorm):
    """Per-head RMSNorm of q and k over the head dim, then RoPE (SWA layers) or
    the SSMax query scale (NoPE layers, keys untouched)  [Attn]. Unrounded."""
    wq, wk = as_f64(w_qnorm), as_f64(w_knorm)
    qn = rms_norm(q, wq, dims.eps)
    kn = rms_norm(k, wk, dims.eps)
    for t, p in enumerate(np.asarray(pos)):
        if mode == "swa":
            qn[t] = rope(qn[t], int(p), dims.theta)
            kn[t] = rope(kn[t], int(p), dims.theta)
        elif mode == "nope":
            qn[t] = qn[t] * ssmax_factor(int(p) + 1)
        else:
            raise ValueError(mode)
    return qn, kn


@dataclass
class KVCache:
    """Logical cache: K[s][j][u][:], V[s][j][u][:] for sequence s, kv head j,
    position u. bf16 caches hold bf16-exact float64 values; fp8 caches hold
    e4m3fn codes with one scale per K cache and one per V cache."""
    K: np.ndarray
    V: np.ndarray
    dtype: str = "bf16"
    k_scale: float = 1.0
    v_scale: float = 1.0

    @classmethod
    def empty(cls, S, Hkv, Lmax, d, dtype="bf16", k_scale=1.0, v_scale=1.0):
        t = F64 if dtype == "bf16" else np.uint8
        return cls(np.zeros((S, Hkv, Lmax, d), t), np.zeros((S, Hkv, Lmax, d), t),
                   dtype, k_scale, v_scale)

    def copy(self):
        return KVCache(self.K.copy(), self.V.copy(), self.dtype, self.k_scale, self.v_scale)

    def store(self, s, j, u, kvec, vvec):
        if self.dtype == "bf16":
            self.K[s, j, u] = bf(kvec)
            self.V[s, j, u] = bf(vvec)
        else:
            self.K[s, j, u] = e4m3_quantize(kvec, self.k_scale)
            self.V[s, j, u] = e4m3_quantize(vvec, self.v_scale)

    def keys(self, s, j, lo, hi):
        """Dequantised keys and values for positions lo..hi inclusive."""
        K, V = self.K[s, j, lo:hi + 1], self.V[s, j, lo:hi + 1]
        if self.dtype == "bf16":
            return K.astype(F64), V.astype(F64)
        return e4m3_decode(K) * self.k_scale, e4m3_decode(V) * self.v_scale


def kv_write(cache: KVCache, k, v, pos, seq):
    """Write each token's post-norm/post-RoPE key and its value into the cache
    at (seq, pos)  ([Opt] item 6: the cache update is fused into the q/k kernel)."""
    for t in range(k.shape[0]):
        for j in range(k.shape[1]):
            cache.store(int(seq[t]), j, int(pos[t]), k[t, j], v[t, j])


def attention(dims, q, pos, seq, cache: KVCache, mode: str, sink=None) -> np.ndarray:
    """GQA attention of bf16 queries over the cache  [Attn].

    Head h reads kv head j = floor(h * Hkv / Hq) (contiguous groups). Token t at
    position p sees keys u in [max(0, p - W + 1), p] on SWA layers (W keys
    including itself) and [0, p] on NoPE layers. Scores are q.k / sqrt(d);
    softmax is max-subtracted. sink (optional, [Flint]) adds exp(sink_h) to the
    softmax denominator only. Output is bf16.
    """
    T = q.shape[0]
    o = np.zeros((T, dims.Hq, dims.d), F64)
    grp = dims.Hq // dims.Hkv
    for t in range(T):
        p = int(pos[t])
        lo = max(0, p - dims.window + 1) if mode == "swa" else 0
        for h in range(dims.Hq):
            j = h // grp
            if h % grp == 0:                      # one fetch per kv head
                K, V = cache.keys(int(seq[t]), j, lo, p)
            z = K @ q[t, h] / math.sqrt(dims.d)
            m = z.max() if sink is None else max(z.max(), float(sink[h]))
            e = np.exp(z - m)
            den = e.sum() + (0.0 if sink is None else math.exp(float(sink[h]) - m))
            o[t, h] = (e / den) @ V
    return bf(o)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, F64)))


def output_gate(dims, o, g, b_gate) -> np.ndarray:
    """z_h = o_h * sigmoid(g_h + b_h): the gate comes from its own full-width
    projection (one value per output element) plus a learned per-head bias,
    broadcast over the head dim  [Attn]."""
    T = o.shape[0]
    gg = np.asarray(g, F64).reshape(T, dims.Hq, dims.d) + as_f64(b_gate)[None, :, None]
    return bf(o * sigmoid(gg)).reshape(T, dims.Hq * dims.d)


def o_proj(z, w_o) -> np.ndarray:
    return bf(np.asarray(z, F64) @ as_f64(w_o).T)


# ----------------------------------------------------------------------------
# FFN half  [MoE]
# ----------------------------------------------------------------------------

def _order(score, idx):
    """Descending by score, ties broken towards the lower index."""
    return np.lexsort((idx, -score))


def router(dims, x, w_r, b_corr=None) -> dict:
    """FP32 router and DeepSeek-V3 grouped selection  [MoE].

    logits = x . W_r^T as a binary32 value (float64 sum, rounded once);
    s = sigmoid(logits) in binary32; s' = s + b_corr (binary32 add; the bias
    steers selection only). Group score = sum of the two largest s' in the
    group; keep the topk_group best groups; take the topk largest s' among
    their experts. Weights = route_scale * s / sum(s) over the selected
    experts, with the unbiased s. Ties go to the lower index; idx is ordered by
    s' descending.

    Also returns the selection margins: the gap between the last kept and the
    first dropped group score, and between the last taken and first passed s'.
    """
    x = as_f64(x)
    T = x.shape[0]
    E, ng, tg, K = dims.E, dims.n_group, dims.topk_group, dims.topk
    gs = E // ng
    logits = (x @ np.asarray(w_r, F64).T).astype(np.float32)
    s = (1.0 / (1.0 + np.exp(-logits.astype(F64)))).astype(np.float32)
    b = np.zeros(E, np.float32) if b_corr is None else np.asarray(b_corr, np.float32)
    sb = (s + b).astype(np.float32)
    idx = np.zeros((T, K), np.int32)
    w = np.zeros((T, K), np.float32)
    gmargin = np.full(T, np.inf)
    emargin = np.full(T, np.inf)
    for t in range(T):
        gscore = np.zeros(ng, np.float32)
        for g in range(ng):
            mem = sb[t, g * gs:(g + 1) * gs]
            top = np.sort(mem)[::-1][:2]
            gscore[g] = top.sum(dtype=np.float32) if top.size == 2 else top[0]
        gorder = _order(gscore.astype(F64), np.arange(ng))
        kept = np.sort(gorder[:tg])
        if tg < ng:
            gmargin[t] = float(gscore[gorder[tg - 1]]) - float(gscore[gorder[tg]])
        cand = np.concatenate([np.arange(g * gs, (g + 1) * gs) for g in kept])
        corder = cand[_order(sb[t, cand].astype(F64), cand)]
        sel = corder[:K]
        if len(corder) > K:
            emargin[t] = float(sb[t, corder[K - 1]]) - float(sb[t, corder[K]])
        idx[t] = sel
        ssel = s[t, sel].astype(F64)
        w[t] = (dims.route_scale * ssel / ssel.sum()).astype(np.float32)
    return dict(logits=logits, s=s, sb=sb, idx=idx, w=w,
                group_margin=gmargin, expert_margin=emargin)


def silu(a):
    a = np.asarray(a, F64)
    return a / (1.0 + np.exp(-a))


def swiglu_ffn(x, w13, w2, F: int) -> tuple[np.ndarray, np.ndarray]:
    """One SwiGLU FFN: u = bf(x W13^T) (rows 0..F-1 gate, F..2F-1 up),
    act = bf(silu(gate) * up), returns (act, act W2^T unrounded)."""
    u = bf(as_f64(x) @ as_f64(w13).T)
    act = bf(silu(u[..., :F]) * u[..., F:])
    return act, act @ as_f64(w2).T


def moe(dims, x, idx, w, get_expert, shared=None) -> np.ndarray:
    """Top-k SwiGLU experts with the weighted combine summed wide, then one
    bf16 rounding  [MoE]. get_expert(e) -> (w13 [2F][D], w2 [D][F]).
    shared: optional (w13, w2) of an always-on expert with weight 1 ([Flint])."""
    x = as_f64(x)
    T = x.shape[0]
    idx = np.asarray(idx)
    acc = np.zeros((T, dims.D), F64)
    # each term w[t][k] * FFN_e(x_t) of the sum, visited expert by expert so
    # every expert's weights are read once
    for e in np.unique(idx):
        w13, w2 = get_expert(int(e))
        tt, kk = np.nonzero(idx == e)
        _, y = swiglu_ffn(x[tt], w13, w2, dims.F)
        for r, (t, k) in enumerate(zip(tt, kk)):
            acc[t] += float(w[t, k]) * y[r]
    if shared is not None:
        _, y = swiglu_ffn(x, shared[0], shared[1], dims.F)
        acc += y
    return bf(acc)


def dense_ffn(x, w13, w2, Fd: int) -> np.ndarray:
    """Dense SwiGLU MLP of the first layers (d_ff 20,480 on Beam)  [MoE]."""
    _, y = swiglu_ffn(x, w13, w2, Fd)
    return bf(y)


# ----------------------------------------------------------------------------
# Output head (after the layer stack)
# ----------------------------------------------------------------------------

def softcap(z, cap: float) -> np.ndarray:
    """cap * tanh(z / cap): the logit soft cap of Beam's output (cap 30; the
    architecture notes of the Chinese digest, "Beam model architecture"
    section). cap = 0 leaves z unchanged."""
    z = np.asarray(z, dtype=F64)
    if cap == 0:
        return z
    return cap * np.tanh(z / cap)


def lm_head_softcap(x, w_head, cap: float) -> np.ndarray:
    """Logits of T final hidden rows: z[t][v] = x[t] . W[v] (W [V][D], the
    LM head's rows), then the soft cap; float64, no rounding (the call
    returns fp32 logits)."""
    return softcap(as_f64(x) @ as_f64(w_head).T, cap)


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------

def layer_forward(dims, params, h_in, pos, seq, cache: KVCache, mode: str, n: int,
                  ffn: str = "moe", get_expert=None, route_override=None,
                  sandwich: bool = True) -> dict:
    """One decoder layer over T tokens (decode: T = 1; chunked prefill: the
    chunk's keys are written before any token attends).

    n is the index of the attention residual add; the FFN add is n + 1.
    The layer entry pre-norm is included (x = rms(h_in; w_attn_pre)).
    sandwich False selects the pre-norm, plain-residual form of [Flint] (no
    post-norms, n ignored). The cache is updated in place (pass a copy).
    route_override replaces the routing indices (weights are recomputed for
    them with the same rule); used to compare near-tie tokens.
    Returns every intermediate.
    """
    r = {}
    P = params
    h0 = as_f64(h_in)
    pos = np.asarray(pos)
    seq = np.asarray(seq)
    _, x = boundary(None, h0, None, P["w_attn_pre"], 0, dims.eps)
    r["x"] = x
    qkvg = qkvg_projection(x, P["w_qkvg"])
    r["qkvg"] = qkvg
    q, k, v, g = split_qkvg(dims, qkvg)
    qn, kn = qk_norm_position(dims, q, k, pos, mode, P["w_qnorm"], P["w_knorm"])
    r["q"] = bf(qn)
    r["k"] = kn
    r["v"] = v
    r["g"] = g
    kv_write(cache, kn, v, pos, seq)
    o = attention(dims, r["q"], pos, seq, cache, mode, sink=P.get("sink"))
    r["o"] = o
    z = output_gate(dims, o, g, P["b_gate"]) if dims.G else o.reshape(o.shape[0], -1)
    r["z"] = z
    y = o_proj(z, P["w_o"])
    r["y"] = y
    if sandwich:
        h1, x2 = boundary(y, h0, P["w_attn_post"], P["w_ffn_pre"], n, dims.eps)
    else:
        h1, x2 = boundary(y, h0, None, P["w_ffn_pre"], 0, dims.eps)
    r["h_mid"], r["x2"] = h1, x2
    if ffn == "moe":
        rt = router(dims, x2, P["w_r"], P.get("b_corr"))
        r.update({"logits": rt["logits"], "s": rt["s"], "idx": rt["idx"], "w": rt["w"],
                  "group_margin": rt["group_margin"], "expert_margin": rt["expert_margin"]})
        idx, w = rt["idx"], rt["w"]
        if route_override is not None:
            idx = np.asarray(route_override, np.int32)
            ssel = np.take_along_axis(rt["s"], idx, axis=1).astype(F64)
            w = (dims.route_scale * ssel / ssel.sum(axis=1, keepdims=True)).astype(np.float32)
        if get_expert is None:
            get_expert = lambda e: (P["w13"][e], P["w2"][e])  # noqa: E731
        shared = (P["shared_w13"], P["shared_w2"]) if dims.shared else None
        y2 = moe(dims, x2, idx, w, get_expert, shared)
    else:
        y2 = dense_ffn(x2, P["dense_w13"], P["dense_w2"], dims.Fd)
    r["y2"] = y2
    if sandwich:
        h2, xn = boundary(y2, h1, P["w_ffn_post"], P["w_next_pre"], n + 1, dims.eps)
    else:
        h2, xn = boundary(y2, h1, None, P["w_next_pre"], 0, dims.eps)
    r["h_out"], r["x_next"] = h2, xn
    return r
