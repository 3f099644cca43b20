"""Pins of the oracle's layer stages against closed forms, library routines
used as special cases, and float64 brute force on the tiny shapes (no GPU).

Each test names the mistake it is there to catch."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import synth
from oracle import accounting, layer as L
from oracle.numerics import round_bf16, bf16_bits_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DIMS0 = synth.config(0).dims


def _tbf(x):
    """torch's bf16 rounding of float64 values that are fp32-exact or not:
    round in float64 -> float32 first is avoided by going through torch's own
    float64 -> bf16 cast."""
    return torch.as_tensor(np.asarray(x, np.float64)).to(torch.bfloat16).double().numpy()


# --------------------------------------------------------------------- RMSNorm
def test_rms_norm_matches_torch_and_unit_rms():
    g = np.random.default_rng(0)
    v = g.standard_normal((7, 256)) * 3.0
    w = g.uniform(0.5, 1.5, 256)
    ref = Fn.rms_norm(torch.tensor(v), (256,), weight=torch.tensor(w), eps=1e-6).numpy()
    np.testing.assert_allclose(L.rms_norm(v, w, 1e-6), ref, rtol=1e-13, atol=0)
    u = L.rms_norm(v, np.ones(256), 1e-6)
    np.testing.assert_allclose(np.sqrt(np.mean(u * u, axis=-1)), 1.0, rtol=1e-6)


# ---------------------------------------------------------- scaled residual
def test_scaled_residual_telescopes():
    """h_n = sqrt(m/n) h_m + (1/sqrt n) sum_{k=m+1..n} x_k  (closed form of the
    recursion h <- sqrt((n-1)/n) h + x/sqrt(n)). Catches a swapped or missing
    sqrt, or (n-1)/n vs n/(n+1) off-by-one."""
    g = np.random.default_rng(1)
    m, n = 7, 30
    h_m = g.standard_normal(64)
    xs = g.standard_normal((n - m, 64))
    h = h_m.copy()
    for k in range(m + 1, n + 1):
        h = L.scaled_residual(h, xs[k - m - 1], k)
    closed = math.sqrt(m / n) * h_m + xs.sum(axis=0) / math.sqrt(n)
    np.testing.assert_allclose(h, closed, rtol=1e-12, atol=1e-12)
    # n = 1 replaces h by x; n = 0 is the plain add
    np.testing.assert_array_equal(L.scaled_residual(h_m, xs[0], 1), xs[0])
    np.testing.assert_allclose(L.scaled_residual(h_m, xs[0], 0), h_m + xs[0])


def test_scaled_residual_keeps_unit_variance():
    """Unit-variance independent sublayer outputs keep the stream at unit
    variance at every depth (the stated purpose of the rule)."""
    g = np.random.default_rng(2)
    h = np.zeros(200000)
    for n in range(1, 105):
        h = L.scaled_residual(h, g.standard_normal(200000), n)
        if n in (1, 2, 10, 104):
            assert abs(h.var() - 1.0) < 0.02, (n, h.var())


def test_boundary_composes_norms_and_residual():
    """Post-norm -> n-th scaled add -> pre-norm with bf16 rounding at each
    stored tensor, rebuilt from torch's rms_norm and bf16 cast."""
    g = np.random.default_rng(3)
    D = 256
    y = _tbf(g.standard_normal((3, D)))
    h = _tbf(g.standard_normal((3, D)))
    wp = _tbf(g.uniform(0.5, 1.5, D))
    wn = _tbf(g.uniform(0.5, 1.5, D))
    n = 21
    a = _tbf(Fn.rms_norm(torch.tensor(y), (D,), torch.tensor(wp), 1e-6).numpy())
    hh = _tbf(math.sqrt(20 / 21) * h + a / math.sqrt(21))
    x = _tbf(Fn.rms_norm(torch.tensor(hh), (D,), torch.tensor(wn), 1e-6).numpy())
    h2, x2 = L.boundary(y, h, wp, wn, n, 1e-6)
    np.testing.assert_array_equal(h2, hh)
    np.testing.assert_array_equal(x2, x)
    h3, x3 = L.boundary(None, h, wp, wn, n, 1e-6)       # layer entry: pre-norm only
    np.testing.assert_array_equal(h3, h)
    np.testing.assert_array_equal(
        x3, _tbf(Fn.rms_norm(torch.tensor(h), (D,), torch.tensor(wn), 1e-6).numpy()))


# --------------------------------------------------------------------- SSMax
def test_ssmax_closed_form_checkpoints():
    """(1 + p/2048)^0.1 = 2^(k/10) exactly at p = 2048 (2^k - 1)."""
    for k in range(1, 8):
        p = 2048 * (2 ** k - 1)
        assert L.ssmax_factor(p) == pytest.approx(2 ** (k / 10), rel=1e-15)
    assert L.ssmax_factor(2048) == pytest.approx(1.0717734625362931, rel=1e-15)
    assert L.ssmax_factor(100001) == pytest.approx(math.exp(0.1 * math.log1p(100001 / 2048)),
                                                   rel=1e-15)
    assert L.ssmax_factor(1) > 1.0 and L.ssmax_factor(1) < 1.0001


# ---------------------------------------------------------------------- RoPE
def _rope_complex(v, pos, theta):
    """Rotation written as complex multiplication of pairs (i, i + d/2)."""
    d = v.shape[-1]
    half = d // 2
    z = v[..., :half] + 1j * v[..., half:]
    z = z * np.exp(1j * pos / theta ** (np.arange(half) * 2.0 / d))
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_matches_complex_rotation_and_invariants():
    g = np.random.default_rng(4)
    q = g.standard_normal((3, 128))
    k = g.standard_normal((3, 128))
    for pos in (0, 1, 17, 100000):
        # angles near 1e5 rad carry ~1e-11 of float64 rounding in either form
        np.testing.assert_allclose(L.rope(q, pos, 1e4), _rope_complex(q, pos, 1e4),
                                   rtol=0, atol=1e-12 * max(1, pos / 100))
    np.testing.assert_array_equal(L.rope(q, 0, 1e4), q)
    r = L.rope(q, 999, 1e4)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(q, axis=-1),
                               rtol=1e-13)
    # <R_a q, R_b k> depends on a - b only
    a, b, dlt = 40, 13, 5000
    lhs = np.sum(L.rope(q, a, 1e4) * L.rope(k, b, 1e4), axis=-1)
    rhs = np.sum(L.rope(q, a + dlt, 1e4) * L.rope(k, b + dlt, 1e4), axis=-1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-9)


def test_qk_norm_then_position():
    """Norm first, then RoPE (SWA) or SSMax on q only (NoPE). Catches norm
    after rotation (differs with a non-uniform gain) and SSMax on keys or at
    the 0-based position."""
    g = np.random.default_rng(5)
    d = DIMS0.d
    q = g.standard_normal((2, DIMS0.Hq, d))
    k = g.standard_normal((2, DIMS0.Hkv, d))
    wq = g.uniform(0.5, 1.5, d)
    wk = g.uniform(0.5, 1.5, d)
    pos = np.array([0, 37])
    tq = Fn.rms_norm(torch.tensor(q), (d,), torch.tensor(wq), DIMS0.eps).numpy()
    tk = Fn.rms_norm(torch.tensor(k), (d,), torch.tensor(wk), DIMS0.eps).numpy()
    qs, ks = L.qk_norm_position(DIMS0, q, k, pos, "swa", wq, wk)
    for t in range(2):
        np.testing.assert_allclose(qs[t], _rope_complex(tq[t], pos[t], DIMS0.theta), atol=1e-12)
        np.testing.assert_allclose(ks[t], _rope_complex(tk[t], pos[t], DIMS0.theta), atol=1e-12)
    qn, kn = L.qk_norm_position(DIMS0, q, k, pos, "nope", wq, wk)
    for t in range(2):
        s = (1 + (pos[t] + 1) / 2048) ** 0.1
        np.testing.assert_allclose(qn[t], tq[t] * s, rtol=1e-13)
        np.testing.assert_allclose(kn[t], tk[t], rtol=1e-13)


# ----------------------------------------------------------------- attention
def _cache_from(K, V):
    return L.KVCache(K.copy(), V.copy(), "bf16")


def _brute_attention(dims, q, pos, K, V, mode):
    """Scores, softmax and weighted sum by explicit loops (float64)."""
    T, Hq, d = q.shape
    grp = Hq // dims.Hkv
    out = np.zeros((T, Hq, d))
    for t in range(T):
        p = int(pos[t])
        lo = max(0, p - dims.window + 1) if mode == "swa" else 0
        for h in range(Hq):
            j = h // grp
            sc = []
            for u in range(lo, p + 1):
                acc = 0.0
                for i in range(d):
                    acc += q[t, h, i] * K[0, j, u, i]
                sc.append(acc / math.sqrt(d))
            mx = max(sc)
            ex = [math.exp(s - mx) for s in sc]
            den = sum(ex)
            for i in range(d):
                out[t, h, i] = sum(ex[n] / den * V[0, j, lo + n, i] for n in range(len(ex)))
    return out


@pytest.mark.parametrize("mode", ["swa", "nope"])
def test_attention_brute_force(mode):
    dims = DIMS0
    g = np.random.default_rng(6)
    Lm = 40
    K = _tbf(g.standard_normal((1, dims.Hkv, Lm, dims.d)))
    V = _tbf(g.standard_normal((1, dims.Hkv, Lm, dims.d)))
    q = _tbf(g.standard_normal((3, dims.Hq, dims.d)))
    pos = np.array([0, 15, 39])
    o = L.attention(dims, q, pos, np.zeros(3, int), _cache_from(K, V), mode)
    ref = _tbf(_brute_attention(dims, q, pos, K, V, mode))
    np.testing.assert_array_equal(o, ref)


def test_attention_special_cases_match_sdpa():
    """W >= pos + 1 makes SWA equal NoPE, and both equal causal SDPA with the
    kv heads repeated over their query groups (contiguous grouping)."""
    dims = synth.with_dims(synth.config(0), window=1000).dims
    g = np.random.default_rng(7)
    Lq = 24
    K = _tbf(g.standard_normal((1, dims.Hkv, Lq, dims.d)))
    V = _tbf(g.standard_normal((1, dims.Hkv, Lq, dims.d)))
    q = _tbf(g.standard_normal((Lq, dims.Hq, dims.d)))
    pos = np.arange(Lq)
    seq = np.zeros(Lq, int)
    o_s = L.attention(dims, q, pos, seq, _cache_from(K, V), "swa")
    o_n = L.attention(dims, q, pos, seq, _cache_from(K, V), "nope")
    np.testing.assert_array_equal(o_s, o_n)
    grp = dims.Hq // dims.Hkv
    kt = torch.tensor(K[0]).repeat_interleave(grp, 0)          # [Hq][L][d]
    vt = torch.tensor(V[0]).repeat_interleave(grp, 0)
    qt = torch.tensor(q).transpose(0, 1)                        # [Hq][L][d]
    ref = Fn.scaled_dot_product_attention(qt, kt, vt, is_causal=True).transpose(0, 1).numpy()
    np.testing.assert_allclose(o_n, _tbf(ref), rtol=0, atol=2 ** -7 * np.abs(ref).max())
    assert np.mean(o_n == _tbf(ref)) > 0.99


def test_attention_degenerate_cases():
    dims = DIMS0
    g = np.random.default_rng(8)
    K = _tbf(g.standard_normal((1, dims.Hkv, 64, dims.d)))
    V = _tbf(g.standard_normal((1, dims.Hkv, 64, dims.d)))
    q = _tbf(g.standard_normal((1, dims.Hq, dims.d)))
    # pos = 0: the single key's value
    o = L.attention(dims, q, [0], [0], _cache_from(K, V), "nope")
    grp = dims.Hq // dims.Hkv
    for h in range(dims.Hq):
        np.testing.assert_array_equal(o[0, h], V[0, h // grp, 0])
    # identical keys: mean of the window's values, exactly W of them
    K2 = np.broadcast_to(K[:, :, :1], K.shape).copy()
    o = L.attention(dims, q, [50], [0], _cache_from(K2, V), "swa")
    for h in range(dims.Hq):
        want = V[0, h // grp, 50 - dims.window + 1:51].mean(axis=0)
        np.testing.assert_allclose(o[0, h], _tbf(want), atol=2 ** -8 * np.abs(want).max())
    # a planted needle key aligned with q dominates
    K3 = K.copy()
    K3[0, 0, 20] = q[0, 0] * 50
    o = L.attention(dims, q, [63], [0], _cache_from(K3, V), "nope")
    np.testing.assert_allclose(o[0, 0], V[0, 0, 20], atol=1e-6)


def test_attention_fp8_cache_dequantises_with_scale():
    dims = DIMS0
    g = np.random.default_rng(9)
    codes_k = g.integers(0, 256, (1, dims.Hkv, 32, dims.d)).astype(np.uint8)
    codes_v = g.integers(0, 256, (1, dims.Hkv, 32, dims.d)).astype(np.uint8)
    for c in (codes_k, codes_v):
        c[(c & 0x7F) == 0x7F] = 0x10                          # no NaN codes
    ks, vs = 0.01, 0.02
    cache = L.KVCache(codes_k, codes_v, "fp8", ks, vs)
    deq = lambda c, s: torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy() * s  # noqa
    ref_cache = _cache_from(deq(codes_k, ks), deq(codes_v, vs))
    q = _tbf(g.standard_normal((1, dims.Hq, dims.d)))
    np.testing.assert_array_equal(L.attention(dims, q, [31], [0], cache, "nope"),
                                  L.attention(dims, q, [31], [0], ref_cache, "nope"))


# ----------------------------------------------------------------- gate
def test_output_gate_limits():
    dims = DIMS0
    g = np.random.default_rng(10)
    o = _tbf(g.standard_normal((2, dims.Hq, dims.d)))
    gg = _tbf(g.standard_normal((2, dims.G)))
    on = L.output_gate(dims, o, gg, np.full(dims.Hq, 1e4))
    np.testing.assert_array_equal(on, o.reshape(2, -1))
    off = L.output_gate(dims, o, gg, np.full(dims.Hq, -1e4))
    np.testing.assert_array_equal(off, 0.0)
    b = g.uniform(-1, 1, dims.Hq)
    ref = o * torch.sigmoid(torch.tensor(gg.reshape(2, dims.Hq, dims.d) + b[None, :, None])).numpy()
    np.testing.assert_array_equal(L.output_gate(dims, o, gg, b), _tbf(ref).reshape(2, -1))


# ----------------------------------------------------------------- router
def _brute_route(dims, logits32, b):
    """Enumerate every set of topk_group groups and every set of topk experts."""
    s = torch.sigmoid(torch.tensor(logits32, dtype=torch.float64)).float().numpy()
    sb = (s + b).astype(np.float32)
    gs = dims.E // dims.n_group
    gscore = [float(np.float32(np.sort(sb[g * gs:(g + 1) * gs])[-2:].sum(dtype=np.float32)))
              for g in range(dims.n_group)]
    best = max(itertools.combinations(range(dims.n_group), dims.topk_group),
               key=lambda c: sum(gscore[i] for i in c))
    cand = [e for g in best for e in range(g * gs, (g + 1) * gs)]
    sel = max(itertools.combinations(cand, dims.topk), key=lambda c: sum(float(sb[e]) for e in c))
    return set(sel), s


def test_router_brute_force_tiny():
    dims = DIMS0
    g = np.random.default_rng(11)
    x = _tbf(g.standard_normal((40, dims.D)))
    w_r = (g.standard_normal((dims.E, dims.D)) * 0.02).astype(np.float32)
    b = g.uniform(-0.1, 0.1, dims.E).astype(np.float32)
    r = L.router(dims, x, w_r, b)
    ref_logits = torch.tensor(x) @ torch.tensor(w_r, dtype=torch.float64).T
    np.testing.assert_allclose(r["logits"], ref_logits.numpy(), rtol=1e-6)
    for t in range(40):
        sel, s = _brute_route(dims, r["logits"][t], b)
        assert set(r["idx"][t].tolist()) == sel
        # weights use the unbiased sigmoid and sum to the route scale
        ws = s[r["idx"][t]].astype(np.float64)
        np.testing.assert_allclose(r["w"][t], 2.5 * ws / ws.sum(), rtol=1e-6)
        assert r["w"][t].sum() == pytest.approx(2.5, rel=1e-6)
        sbs = r["sb"][t][r["idx"][t]]
        assert np.all(np.diff(sbs) <= 0)                        # ordered by s' descending


def test_router_single_group_is_topk():
    dims = synth.with_dims(synth.config(0), n_group=1, topk_group=1).dims
    g = np.random.default_rng(12)
    x = _tbf(g.standard_normal((20, dims.D)))
    w_r = (g.standard_normal((dims.E, dims.D)) * 0.02).astype(np.float32)
    b = g.uniform(-0.1, 0.1, dims.E).astype(np.float32)
    r = L.router(dims, x, w_r, b)
    ref = torch.topk(torch.tensor(r["sb"]), dims.topk, dim=1).indices.numpy()
    np.testing.assert_array_equal(r["idx"], ref)
    r0 = L.router(dims, x, w_r, None)                            # no bias: top-k of logits
    np.testing.assert_array_equal(r0["idx"],
                                  torch.topk(torch.tensor(r0["logits"]), dims.topk, 1).indices)


def test_router_ties_lower_index():
    dims = DIMS0
    x = np.ones((1, dims.D))
    w_r = np.zeros((dims.E, dims.D), np.float32)               # all scores equal
    r = L.router(dims, x, w_r, None)
    # groups 0 and 1 kept, then experts 0..3
    assert r["idx"][0].tolist() == [0, 1, 2, 3]
    assert r["group_margin"][0] == 0 and r["expert_margin"][0] == 0


# ----------------------------------------------------------------- experts
def test_moe_equals_dense_of_concatenated_experts():
    """Dense FFN whose W13/W2 concatenate k experts' weights equals the MoE
    over those experts at weight 1 (d_ff 20480 = 8 x 2560 makes this exact on
    Beam). Catches a transposed W2, a swapped gate/up half, or a combine that
    skips or double-counts an expert."""
    dims = DIMS0
    p = synth.make_params(dims, 0, 2)
    g = np.random.default_rng(13)
    x = _tbf(g.standard_normal((5, dims.D)))
    sel = [3, 7, 1, 12]
    F = dims.F
    w13 = np.concatenate([p["w13"][e][:F] for e in sel] + [p["w13"][e][F:] for e in sel])
    w2 = np.concatenate([p["w2"][e] for e in sel], axis=1)
    dense = L.dense_ffn(x, w13, w2, F * len(sel))
    idx = np.tile(np.array(sel, np.int32), (5, 1))
    moe = L.moe(dims, x, idx, np.ones((5, 4), np.float32), lambda e: (p["w13"][e], p["w2"][e]))
    ulp = 2.0 ** (np.floor(np.log2(np.abs(dense) + 1e-30)) - 7)
    assert np.all(np.abs(moe - dense) <= ulp)
    assert np.mean(moe == dense) > 0.99


def test_swiglu_matches_torch():
    dims = DIMS0
    p = synth.make_params(dims, 0, 2)
    x = _tbf(np.random.default_rng(14).standard_normal((3, dims.D)))
    w13 = bf16_bits_to_f64(p["w13"][5])
    w2 = bf16_bits_to_f64(p["w2"][5])
    u = _tbf(torch.tensor(x) @ torch.tensor(w13).T)
    act = _tbf(Fn.silu(torch.tensor(u[:, :dims.F])).numpy() * u[:, dims.F:])
    act_o, y = L.swiglu_ffn(x, p["w13"][5], p["w2"][5], dims.F)
    np.testing.assert_array_equal(act_o, act)
    np.testing.assert_allclose(y, act @ w2.T, rtol=1e-12)
    # one expert at weight 1 is the dense FFN
    moe1 = L.moe(synth.with_dims(synth.config(0), topk=1).dims, x, np.full((3, 1), 5, np.int32),
                 np.ones((3, 1), np.float32), lambda e: (p["w13"][e], p["w2"][e]))
    np.testing.assert_array_equal(moe1, L.dense_ffn(x, p["w13"][5], p["w2"][5], dims.F))


# ----------------------------------------------------------------- accounting
def test_kv_footprint_and_schedule_match_printed_values():
    gold = json.load(open(os.path.join(GOLDEN, "kv_footprint.json")))
    b = gold["beam"]
    assert b["n_full_layers"] * 2 * b["n_kv_heads"] * b["head_dim"] == b["values_per_token"]
    assert accounting.kv_bytes_per_token(9, 8, 128, 2) == b["bf16_KiB_per_token"] * 1024
    assert accounting.kv_bytes_per_token(9, 8, 128, 1) == b["fp8_KiB_per_token"] * 1024
    assert accounting.kv_bytes_per_token(9, 8, 128, 1) * 2 ** 20 == b["fp8_GiB_1M_tokens"] * 2 ** 30
    f = gold["flint"]
    assert accounting.kv_bytes_per_token(14, 4, 128, 2) == f["bf16_KiB_per_token"] * 1024
    s = gold["beam_schedule"]
    nope = accounting.nope_layers(s["layers"])
    assert len(nope) == s["nope_layers"] and s["layers"] - len(nope) == s["swa_layers"]
    assert nope == [5, 11, 17, 23, 29, 35, 41, 47, 51]
    kinds = [accounting.layer_kind(l) for l in range(s["layers"])]
    assert sum(k[1] == "dense" for k in kinds) == s["dense_layers"]
    assert sum(k[1] == "moe" for k in kinds) == s["moe_layers"]
    assert accounting.n_boundaries() == s["boundaries"]
    assert accounting.residual_indices(10) == (21, 22)


# ----------------------------------------------------------------- whole layer
def _tiny_layer(mode, T, pos0, cache=None, h=None, seed=0):
    cfg = synth.config(0)
    dims = cfg.dims
    p = synth.make_params(dims, seed, cfg.extra["layer"])
    if cache is None:
        K, V, _, _ = synth.make_kv_prior(dims, 1, cfg.extra["ctx"], "bf16", seed, 2)
        cache = L.KVCache.empty(1, dims.Hkv, cfg.extra["Lmax"], dims.d)
        cache.K[:, :, :cfg.extra["ctx"]] = bf16_bits_to_f64(K)
        cache.V[:, :, :cfg.extra["ctx"]] = bf16_bits_to_f64(V)
    pos = np.arange(pos0, pos0 + T)
    r = L.layer_forward(dims, p, h, pos, np.zeros(T, int), cache, mode, cfg.extra["n"])
    return r, cache


@pytest.mark.parametrize("mode", ["swa", "nope"])
def test_chunking_invariance(mode):
    """prefill(a+b) == prefill(a) then prefill(b) == prefill(a) then b decodes."""
    h = synth.make_h((12, DIMS0.D), 0, "chunk")
    full, _ = _tiny_layer(mode, 12, 64, h=h)
    c1, cache = _tiny_layer(mode, 8, 64, h=h[:8])
    c2, _ = _tiny_layer(mode, 4, 72, cache=cache, h=h[8:])
    two = np.concatenate([c1["h_out"], c2["h_out"]])
    _, cache = _tiny_layer(mode, 8, 64, h=h[:8])
    dec = []
    for i in range(4):
        r, cache = _tiny_layer(mode, 1, 72 + i, cache=cache, h=h[8 + i:9 + i])
        dec.append(r["h_out"])
    dec = np.concatenate([c1["h_out"]] + dec)
    for other in (two, dec):
        ulp = 2.0 ** (np.floor(np.log2(np.abs(full["h_out"]) + 1e-30)) - 7)
        assert np.all(np.abs(other - full["h_out"]) <= ulp)


def test_tiny_layer_runs_and_normalises():
    h = synth.make_h((2, DIMS0.D), 0, "run")
    r, _ = _tiny_layer("nope", 2, 64, h=h)
    for key in ("x", "q", "o", "y", "h_mid", "x2", "y2", "h_out", "x_next"):
        assert np.all(np.isfinite(r[key])), key
    w = bf16_bits_to_f64(synth.make_params(DIMS0, 0, 2)["w_next_pre"])
    # x_next = rms(h_out) * w, so x_next / w has unit RMS
    u = r["x_next"] / w
    np.testing.assert_allclose(np.sqrt(np.mean(u * u, axis=-1)), 1.0, rtol=1e-2)


# ------------------------------------------- second model: sink, shared expert, pre-norm
# Flint page, "Flint model architecture": a learned attention-sink logit per
# head, one always-on shared expert beside the routed ones, and the plain
# pre-norm residual. Each pin below also evaluates the forms a plausible
# mistake would produce and checks that the pin tells them apart.

def _sink_loops(dims, q, pos, K, V, mode, sink):
    """Softmax with one extra logit per head in the denominator only, by
    explicit loops and without max subtraction (inputs keep exponents small):
    o = sum_u e^{z_u} v_u / (sum_u e^{z_u} + e^{sink_h}).
    Also returns two wrong forms: the sink's term added to every numerator
    element as well (a sink key whose value is all ones), and the sink's term
    left unshifted after the keys' own max is subtracted."""
    T, Hq, d = q.shape
    grp = Hq // dims.Hkv
    good = np.zeros((T, Hq, d))
    numer = np.zeros((T, Hq, d))
    unshift = np.zeros((T, Hq, d))
    for t in range(T):
        p = int(pos[t])
        lo = max(0, p - dims.window + 1) if mode == "swa" else 0
        for h in range(Hq):
            j = h // grp
            ez = []
            for u in range(lo, p + 1):
                acc = 0.0
                for i in range(d):
                    acc += q[t, h, i] * K[0, j, u, i]
                ez.append(math.exp(acc / math.sqrt(d)))
            es = math.exp(float(sink[h]))
            den = sum(ez) + es
            zmax = max(math.log(e) for e in ez)
            den_unshift = sum(e / math.exp(zmax) for e in ez) + es
            for i in range(d):
                num = sum(ez[n] * V[0, j, lo + n, i] for n in range(len(ez)))
                good[t, h, i] = num / den
                numer[t, h, i] = (num + es) / den
                unshift[t, h, i] = num / math.exp(zmax) / den_unshift
    return good, numer, unshift


def _ulp_close(got, ref, ulps=1):
    """Every element within `ulps` bf16 ulps of ref (float64 vs bf16-rounded)."""
    u = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), np.abs(got)) + 1e-300)) - 7)
    return np.all(np.abs(got - ref) <= ulps * u)


@pytest.mark.parametrize("mode", ["swa", "nope"])
def test_attention_sink_brute_force(mode):
    """The sink adds e^{sink} to the denominator only. Catches a sink term in
    the numerator, a sink exponent not shifted by the subtracted max, and a
    sink on the wrong head."""
    dims = synth.with_dims(synth.config(0), sink=True).dims
    g = np.random.default_rng(31)
    Lm = 40
    K = _tbf(g.standard_normal((1, dims.Hkv, Lm, dims.d)))
    V = _tbf(g.standard_normal((1, dims.Hkv, Lm, dims.d)))
    q = _tbf(g.standard_normal((3, dims.Hq, dims.d)) * 2.0)   # scores spread well off 0
    pos = np.array([0, 15, 39])
    sink = np.array([0.5, -1.0, 2.0, 3.5])
    o = L.attention(dims, q, pos, np.zeros(3, int), _cache_from(K, V), mode, sink=sink)
    good, numer, unshift = _sink_loops(dims, q, pos, K, V, mode, sink)
    assert _ulp_close(o, good)
    assert np.mean(o == _tbf(good)) > 0.99
    for wrong in (numer, unshift):
        assert not _ulp_close(o, wrong, ulps=4)
    # per-head: the same sinks in another head order change the result
    o_perm = L.attention(dims, q, pos, np.zeros(3, int), _cache_from(K, V), mode,
                         sink=sink[::-1].copy())
    assert not _ulp_close(o, o_perm, ulps=4)


def test_attention_sink_limits_and_closed_forms():
    dims = synth.with_dims(synth.config(0), sink=True).dims
    g = np.random.default_rng(32)
    K = _tbf(g.standard_normal((1, dims.Hkv, 64, dims.d)))
    V = _tbf(g.standard_normal((1, dims.Hkv, 64, dims.d)))
    q = _tbf(g.standard_normal((2, dims.Hq, dims.d)) * 2.0)
    cache = _cache_from(K, V)
    pos = np.array([9, 50])
    seq = np.zeros(2, int)
    # sink -> -inf leaves exactly the sink-free attention
    for mode in ("swa", "nope"):
        np.testing.assert_array_equal(
            L.attention(dims, q, pos, seq, cache, mode, sink=np.full(dims.Hq, -1e30)),
            L.attention(dims, q, pos, seq, cache, mode))
    # sink -> +inf: every key's weight vanishes
    big = L.attention(dims, q, pos, seq, cache, "nope", sink=np.full(dims.Hq, 200.0))
    assert np.all(np.abs(big) < 1e-60)
    # one key (position 0): o = v0 e^z / (e^z + e^s) = v0 * sigmoid(z - s)
    grp = dims.Hq // dims.Hkv
    sink = np.array([-2.0, 0.0, 1.5, 4.0])
    o = L.attention(dims, q[:1], [0], [0], cache, "nope", sink=sink)
    for h in range(dims.Hq):
        z = float(q[0, h] @ K[0, h // grp, 0]) / math.sqrt(dims.d)
        want = V[0, h // grp, 0] / (1.0 + math.exp(sink[h] - z))
        assert _ulp_close(o[0, h], want)
        # the wrong forms: sink in the numerator, or its exponent unshifted
        wrong_num = (V[0, h // grp, 0] * math.exp(z) + math.exp(sink[h])) / \
            (math.exp(z) + math.exp(sink[h]))
        wrong_unshift = V[0, h // grp, 0] / (1.0 + math.exp(sink[h]))
        assert not _ulp_close(o[0, h], wrong_num, ulps=4)
        assert not _ulp_close(o[0, h], wrong_unshift, ulps=4)
    # n identical keys of score z: o = (sum of their values) e^z / (n e^z + e^s)
    K2 = np.broadcast_to(K[:, :, :1], K.shape).copy()
    o = L.attention(dims, q[:1], [30], [0], _cache_from(K2, V), "swa", sink=sink)
    lo = 30 - dims.window + 1
    n = dims.window
    for h in range(dims.Hq):
        z = float(q[0, h] @ K2[0, h // grp, 0]) / math.sqrt(dims.d)
        want = V[0, h // grp, lo:31].sum(axis=0) * math.exp(z) / (n * math.exp(z) +
                                                                  math.exp(sink[h]))
        assert _ulp_close(o[0, h], want)


def _torch_swiglu(x, w13_bits, w2_bits, F):
    """SwiGLU FFN through torch: bf16 after the gate/up product, after the
    activation, and after the down product."""
    w13 = torch.tensor(bf16_bits_to_f64(w13_bits))
    w2 = torch.tensor(bf16_bits_to_f64(w2_bits))
    u = torch.tensor(_tbf((torch.tensor(x) @ w13.T).numpy()))
    act = torch.tensor(_tbf((Fn.silu(u[:, :F]) * u[:, F:]).numpy()))
    return act @ w2.T


def test_moe_shared_expert_pins():
    """The shared expert is one more SwiGLU expert at weight exactly 1, added
    for every token beside the routed ones. Pinned three ways: all routed
    weights 0 gives torch's SwiGLU of the shared expert alone; at routed
    weight 1 the MoE equals one dense FFN over the concatenated routed and
    shared weights; at routed weights w the dense FFN with each expert's down
    projection scaled by its weight (shared unscaled) gives the same sum.
    Catches a shared weight other than 1, a shared term scaled by a routed
    weight or the route scale, and a shared term that is skipped."""
    dims = synth.with_dims(synth.config(0), shared=True).dims
    p = synth.make_params(dims, 0, 2)
    F = dims.F
    g = np.random.default_rng(33)
    T = 5
    x = _tbf(g.standard_normal((T, dims.D)))
    sel = [3, 7, 1, 12]
    idx = np.tile(np.array(sel, np.int32), (T, 1))
    get = lambda e: (p["w13"][e], p["w2"][e])  # noqa: E731
    sh = (p["shared_w13"], p["shared_w2"])
    y_sh = _torch_swiglu(x, sh[0], sh[1], F).numpy()
    # routed weights 0: the shared expert alone
    m0 = L.moe(dims, x, idx, np.zeros((T, 4), np.float32), get, shared=sh)
    assert _ulp_close(m0, y_sh) and np.mean(m0 == _tbf(y_sh)) > 0.99
    # routed weights 1: one dense FFN over the concatenated five experts
    all13 = [p["w13"][e] for e in sel] + [sh[0]]
    all2 = [p["w2"][e] for e in sel] + [sh[1]]
    w13 = np.concatenate([a[:F] for a in all13] + [a[F:] for a in all13])
    w2 = np.concatenate(all2, axis=1)
    dense = L.dense_ffn(x, w13, w2, F * 5)
    m1 = L.moe(dims, x, idx, np.ones((T, 4), np.float32), get, shared=sh)
    assert _ulp_close(m1, dense) and np.mean(m1 == dense) > 0.99
    # routed weights w: scale each routed expert's down projection by its weight
    w = g.uniform(0.1, 1.2, (T, 4)).astype(np.float32)
    for t in range(T):
        w2s = np.concatenate([bf16_bits_to_f64(p["w2"][e]) * float(w[t, k])
                              for k, e in enumerate(sel)] + [bf16_bits_to_f64(sh[1])], axis=1)
        d_t = L.dense_ffn(x[t:t + 1], w13, w2s, F * 5)
        m_t = L.moe(dims, x[t:t + 1], idx[t:t + 1], w[t:t + 1], get, shared=sh)
        assert _ulp_close(m_t, d_t)
    # the wrong forms differ from the pinned value by many ulps
    routed = L.moe(dims, x, idx, np.ones((T, 4), np.float32), get)
    for k in (0.0, 2.0, 2.5):
        assert not _ulp_close(m1, _tbf(routed + k * y_sh), ulps=4)


def test_prenorm_layer_form():
    """layer_forward(sandwich=False): the pre-norm, plain-residual layer of
    the second model: h_mid = h + y and h_out = h_mid + y2 with no post-norm,
    each bf16; the next sublayer's input is the RMS norm of the residual.
    Rebuilt from the layer's own intermediates with torch's rms_norm and
    bf16 cast. Catches a post-norm that is still applied, a depth-scaled add,
    and the residual index leaking into the plain add."""
    cfg = synth.config(0)
    dims = cfg.dims
    p = synth.make_params(dims, 0, cfg.extra["layer"])
    K, V, _, _ = synth.make_kv_prior(dims, 1, cfg.extra["ctx"], "bf16", 0, 2)

    def run(params, n, sandwich):
        cache = L.KVCache.empty(1, dims.Hkv, cfg.extra["Lmax"], dims.d)
        cache.K[:, :, :cfg.extra["ctx"]] = bf16_bits_to_f64(K)
        cache.V[:, :, :cfg.extra["ctx"]] = bf16_bits_to_f64(V)
        h = synth.make_h((3, dims.D), 0, "prenorm")
        return L.layer_forward(dims, params, h, np.arange(64, 67), np.zeros(3, int), cache,
                               "swa", n, sandwich=sandwich), bf16_bits_to_f64(h)

    r, h = run(p, cfg.extra["n"], False)
    D = dims.D
    rn = lambda v, w: Fn.rms_norm(torch.tensor(v), (D,), torch.tensor(bf16_bits_to_f64(w)),  # noqa
                                  dims.eps).numpy()
    np.testing.assert_array_equal(r["h_mid"], _tbf(h + r["y"]))
    np.testing.assert_array_equal(r["x2"], _tbf(rn(r["h_mid"], p["w_ffn_pre"])))
    np.testing.assert_array_equal(r["h_out"], _tbf(r["h_mid"] + r["y2"]))
    np.testing.assert_array_equal(r["x_next"], _tbf(rn(r["h_out"], p["w_next_pre"])))
    # the post-norm gains and the residual index play no part
    p2 = dict(p)
    p2["w_attn_post"] = None
    p2["w_ffn_post"] = None
    r2, _ = run(p2, 1, False)
    for k in ("h_mid", "x2", "h_out", "x_next"):
        np.testing.assert_array_equal(r2[k], r[k])
    # and the sandwich form is a different layer
    rs, _ = run(p, cfg.extra["n"], True)
    assert not np.array_equal(rs["h_out"], r["h_out"])
