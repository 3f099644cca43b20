"""Seeded synthetic inputs for the Beam decoder layer: shapes, weights, residual
streams and prior KV caches.

This module draws numbers and shapes only. It holds none of the layer's
arithmetic: rounding to bf16 and to fp8 e4m3 is delegated to torch's own dtype
casts (library conversions), so that neither the oracle nor the HIP path
supplies any of the bytes both are fed.

Distributions (the pages run their microbenchmarks on dummy weights; the
choices below are test-data choices, stated once here):
  * projection / expert / dense weights  N(0, 0.02) drawn in fp32, cast to bf16
  * router weight W_r                    N(0, 0.02) fp32;  correction bias U(-0.1, 0.1) fp32
  * gate bias                             U(-1, 1) -> bf16
  * norm gains                            U(0.5, 1.5) -> bf16  (a dropped gain is visible)
  * residual stream h                     N(0, 1) -> bf16
  * prior keys / values                   N(0, 1) -> bf16, or -> fp8 e4m3 with a
                                          per-tensor scale amax/448
Each tensor has its own PCG64 stream keyed by (seed, layer, name, expert), so
one expert can be regenerated without the others.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = [
    "Dims", "CONFIGS", "config", "rng", "bf16_bits_from_f32", "normal_bf16",
    "uniform_bf16", "make_params", "make_expert", "make_dense", "make_h",
    "make_kv_prior",
]


@dataclass(frozen=True)
class Dims:
    D: int
    Hq: int
    Hkv: int
    d: int
    G: int
    E: int
    n_group: int
    topk_group: int
    topk: int
    F: int
    window: int
    Fd: int = 0
    eps: float = 1e-6
    route_scale: float = 2.5
    theta: float = 1e4
    shared: bool = False        # one always-on shared expert (second model only)
    sink: bool = False          # learned per-head attention sink (second model only)

    @property
    def qkvg_rows(self) -> int:
        return self.Hq * self.d + 2 * self.Hkv * self.d + self.G


@dataclass(frozen=True)
class Config:
    name: str
    dims: Dims
    extra: dict = field(default_factory=dict)


_BEAM = Dims(D=5120, Hq=48, Hkv=8, d=128, G=6144, E=256, n_group=8, topk_group=4,
             topk=8, F=2560, window=512, Fd=20480)

CONFIGS = {
    # tiny layer: every shape small enough for float64 brute force
    0: Config("tiny", Dims(D=256, Hq=4, Hkv=2, d=32, G=128, E=16, n_group=4,
                           topk_group=2, topk=4, F=64, window=16, Fd=512),
              dict(layer=2, n=5, ctx=64, prefill=32, Lmax=128)),
    # SWA MoE layer 10, batch-1 decode, bf16 KV holding 100K tokens
    1: Config("beam_swa_decode", _BEAM,
              dict(layer=10, n=21, pos=100000, Lmax=100352, kv="bf16", mode="swa")),
    # NoPE MoE layer 11, batch-1 decode at 100K context, fp8 e4m3 KV
    2: Config("beam_nope_fp8_decode", _BEAM,
              dict(layer=11, n=23, pos=100000, Lmax=100352, kv="fp8", mode="nope")),
    # chunked prefill, 8 x 2048 new tokens on 100K prior, bf16 KV
    3: Config("beam_prefill", _BEAM,
              dict(S=8, chunk=2048, prior=100000, Lmax=102400, kv="bf16",
                   layers={"nope_moe": 11, "swa_moe": 10, "dense": 0})),
    # second model's shape: batch-128 decode, 8K context per sequence
    4: Config("flint_b128_decode",
              Dims(D=2048, Hq=32, Hkv=4, d=128, G=0, E=256, n_group=1, topk_group=1,
                   topk=6, F=512, window=513, route_scale=1.0, shared=True, sink=True),
              dict(B=128, ctx=8192, Lmax=8448, kv="bf16")),
}


def config(i: int) -> Config:
    return CONFIGS[i]


def _key(*parts) -> int:
    return zlib.crc32("/".join(str(p) for p in parts).encode())


def rng(seed: int, *key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _key(*key)])))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """torch's fp32 -> bf16 cast; returns the raw 16-bit patterns as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, std, seed, *key) -> np.ndarray:
    g = rng(seed, *key)
    return bf16_bits_from_f32(g.standard_normal(shape, dtype=np.float32) * np.float32(std))


def uniform_bf16(shape, lo, hi, seed, *key) -> np.ndarray:
    g = rng(seed, *key)
    return bf16_bits_from_f32(g.uniform(lo, hi, shape).astype(np.float32))


def make_expert(dims: Dims, seed: int, layer: int, e, F: int | None = None):
    """(w13 [2F][D] bf16 bits: gate rows then up rows, w2 [D][F] bf16 bits)."""
    F = dims.F if F is None else F
    w13 = normal_bf16((2 * F, dims.D), 0.02, seed, layer, "w13", e)
    w2 = normal_bf16((dims.D, F), 0.02, seed, layer, "w2", e)
    return w13, w2


def make_dense(dims: Dims, seed: int, layer: int):
    return make_expert(dims, seed, layer, "dense", F=dims.Fd)


def make_params(dims: Dims, seed: int, layer: int, experts: bool = True,
                dense: bool = False, projections: bool = True) -> dict:
    """All small per-layer tensors, plus every expert when experts=True.

    Gains for the layer's four sandwich norms and the next layer's pre-norm,
    q/k norm gains, the packed [q | k | v | g] projection, gate bias, o_proj,
    fp32 router weight and correction bias.
    """
    D, d = dims.D, dims.d
    p = {}
    for name in ("w_attn_pre", "w_attn_post", "w_ffn_pre", "w_ffn_post", "w_next_pre"):
        p[name] = uniform_bf16((D,), 0.5, 1.5, seed, layer, name)
    p["w_qnorm"] = uniform_bf16((d,), 0.5, 1.5, seed, layer, "w_qnorm")
    p["w_knorm"] = uniform_bf16((d,), 0.5, 1.5, seed, layer, "w_knorm")
    if projections:
        p["w_qkvg"] = normal_bf16((dims.qkvg_rows, D), 0.02, seed, layer, "w_qkvg")
        p["w_o"] = normal_bf16((D, dims.Hq * d), 0.02, seed, layer, "w_o")
    if dims.G:
        p["b_gate"] = uniform_bf16((dims.Hq,), -1.0, 1.0, seed, layer, "b_gate")
    g = rng(seed, layer, "w_r")
    p["w_r"] = (g.standard_normal((dims.E, D), dtype=np.float32) * np.float32(0.02))
    g = rng(seed, layer, "b_corr")
    p["b_corr"] = g.uniform(-0.1, 0.1, dims.E).astype(np.float32)
    if dims.sink:
        g = rng(seed, layer, "sink")
        p["sink"] = g.standard_normal(dims.Hq).astype(np.float32)
    if experts:
        w13 = np.empty((dims.E, 2 * dims.F, D), np.uint16)
        w2 = np.empty((dims.E, D, dims.F), np.uint16)
        for e in range(dims.E):
            w13[e], w2[e] = make_expert(dims, seed, layer, e)
        p["w13"], p["w2"] = w13, w2
        if dims.shared:
            p["shared_w13"], p["shared_w2"] = make_expert(dims, seed, layer, "shared")
    if dense:
        p["dense_w13"], p["dense_w2"] = make_dense(dims, seed, layer)
    return p


def make_h(shape, seed: int, *key) -> np.ndarray:
    """Residual stream / activations: N(0, 1) cast to bf16 (uint16 bits)."""
    return normal_bf16(shape, 1.0, seed, "h", *key)


def make_kv_prior(dims: Dims, S: int, ctx: int, kv: str, seed: int, layer: int):
    """Prior cache contents in logical order K[s][j][u][:], V[s][j][u][:], u < ctx.

    kv == "bf16": returns (K bits, V bits, 1.0, 1.0) as uint16.
    kv == "fp8":  returns (K codes, V codes, k_scale, v_scale) as uint8 e4m3fn
                  codes with per-tensor scales amax/448 of the drawn values.
    """
    g = rng(seed, layer, "kv_prior")
    K = g.standard_normal((S, dims.Hkv, ctx, dims.d), dtype=np.float32)
    V = g.standard_normal((S, dims.Hkv, ctx, dims.d), dtype=np.float32)
    if kv == "bf16":
        return bf16_bits_from_f32(K), bf16_bits_from_f32(V), 1.0, 1.0
    if kv == "fp8":
        out = []
        for a in (K, V):
            scale = float(np.abs(a).max()) / 448.0
            t = torch.from_numpy(a / np.float32(scale)).clamp_(-448.0, 448.0)
            out.append(t.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
            out.append(scale)
        return out[0], out[2], out[1], out[3]
    raise ValueError(kv)


def with_dims(cfg: Config, **kw) -> Config:
    return replace(cfg, dims=replace(cfg.dims, **kw))


# ---------------------------------------------------------------------------
# Full-size tensors are drawn on the device with torch's counter-based
# generator (seeded from the same key scheme); the oracle reads back only the
# slices it needs.
def _torch_gen(seed: int, key, device):
    g = torch.Generator(device=device)
    g.manual_seed(((seed & 0xFFFFFFFF) << 32) ^ _key(*key))
    return g


def torch_normal_bf16(shape, std, seed, *key, device="cuda", out=None):
    """N(0, std) drawn in fp32 on `device`, cast to bf16; returned as int16 bits."""
    g = _torch_gen(seed, key, device)
    t = (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std)
    t = t.to(torch.bfloat16).view(torch.int16)
    if out is not None:
        out.copy_(t)
        return out
    return t


def torch_uniform_bf16(shape, lo, hi, seed, *key, device="cuda"):
    g = _torch_gen(seed, key, device)
    t = torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo
    return t.to(torch.bfloat16).view(torch.int16)


def torch_kv_prior(dims: Dims, S: int, ctx: int, kv: str, seed: int, layer: int, device="cuda"):
    """Device version of make_kv_prior: logical K, V [S][Hkv][ctx][d] as int16 bf16
    bits or uint8 e4m3fn codes, plus the two scales."""
    out = []
    for name in ("k", "v"):
        g = _torch_gen(seed, (layer, "kv_prior", name), device)
        a = torch.randn((S, dims.Hkv, ctx, dims.d), generator=g, device=device,
                        dtype=torch.float32)
        if kv == "bf16":
            out += [a.to(torch.bfloat16).view(torch.int16), 1.0]
        else:
            scale = float(a.abs().max()) / 448.0
            q = (a / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
            out += [q, scale]
        del a
    return out[0], out[2], out[1], out[3]
