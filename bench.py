"""Benchmark: Beam SWA MoE decoder layer, batch-1 decode at 100K context, one
MI355X.

A step is one full layer-step of the hot path through the C ABI:
  packed QKVG projection + q/k norm + RoPE + KV write -> SWA attention over
  512 keys of a 100K-token bf16 cache -> sigmoid gate + o_proj -> boundary
  (post-norm, depth-scaled residual, pre-norm) -> FP32 router + grouped top-8
  -> 8 SwiGLU experts + combine -> boundary.
Steps are chained as in a layer stack: step i's residual output and next
pre-norm feed step i+1, and consecutive steps alternate between two full,
distinct layer weight sets (2 x 21 GB, each with all 256 experts), so weights
stream from HBM rather than the 256 MB Infinity Cache. A chain of steps is
captured in one HIP graph and replayed; the timed region holds exactly
--steps steps.

Prints one JSON line (rank 0). --gpus above 1 exits: the layer runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, GB/s (published)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--chain", type=int, default=8, help="layer-steps per captured graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-nope", action="store_true", help="skip the NoPE fp8 decode leg")
    ap.add_argument("--no-flint", action="store_true",
                    help="skip the second model's batch-128 decode legs")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the SWA decode legs with block-scaled (MXFP8, MXFP4) experts")
    ap.add_argument("--no-1m", action="store_true",
                    help="skip the NoPE fp8 decode leg at a 2^20-token context")
    ap.add_argument("--no-head", action="store_true",
                    help="skip the output head (logit soft cap) leg")
    ap.add_argument("--no-mx-prefill", action="store_true",
                    help="skip the prefill MoE leg on block-scaled operands")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 52-layer decode step at a 2^20-token context")
    ap.add_argument("--stack-steps", type=int, default=10,
                    help="timed whole-model decode steps (each about 14 ms)")
    ap.add_argument("--unfused", action="store_true",
                    help="batch-1 decode legs with the separate q/k, attention and gate + "
                         "o_proj calls instead of the fused attention call")
    ap.add_argument("--prefill-reps", type=int, default=3)
    ap.add_argument("--cpu-steps", type=int, default=8)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB copy kernel (HBM counter calibration)")
    ap.add_argument("--counters", action="store_true",
                    help="only launch the expert gate/up kernel, eagerly, 20 times "
                         "(a short program for rocprofv3 --pmc passes)")
    ap.add_argument("--counters-step", action="store_true",
                    help="only run 8 decode layer-steps of the SWA layer eagerly (every "
                         "kernel of the step, for rocprofv3 --pmc passes)")
    ap.add_argument("--counters-prefill", action="store_true",
                    help="only run one pass of each prefill layer eagerly (for rocprofv3 "
                         "--pmc passes)")
    ap.add_argument("--counters-mx", choices=["bf16", "mxfp8", "mxfp4"],
                    help="only run the prefill MoE once with the given expert format "
                         "(for rocprofv3 --pmc passes)")
    return ap.parse_args()


# ----------------------------------------------------------------------------
class LayerSet:
    """One layer's weights and KV cache on the device (random-init, seeded)."""

    def __init__(self, dims, seed, layer, ctx, Lmax, kv="bf16", experts="bf16"):
        import numpy as np
        import torch

        import moe_decoder_layer_amd as B
        import synth
        self.dims = dims
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(  # noqa: E731
            a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
        p = synth.make_params(dims, seed, layer, experts=False, projections=False)
        self.t = {k: dev(v) for k, v in p.items()}
        self.t["w_qkvg"] = synth.torch_normal_bf16((dims.qkvg_rows, dims.D), 0.02, seed, layer,
                                                   "w_qkvg")
        self.t["w_o"] = synth.torch_normal_bf16((dims.D, dims.Hq * dims.d), 0.02, seed, layer,
                                                "w_o")
        w13 = torch.empty((dims.E, 2 * dims.F, dims.D), dtype=torch.int16, device="cuda")
        w2 = torch.empty((dims.E, dims.D, dims.F), dtype=torch.int16, device="cuda")
        for e in range(dims.E):
            synth.torch_normal_bf16((2 * dims.F, dims.D), 0.02, seed, layer, "w13", e, out=w13[e])
            synth.torch_normal_bf16((dims.D, dims.F), 0.02, seed, layer, "w2", e, out=w2[e])
        self.t["w13"], self.t["w2"] = w13, w2
        if experts != "bf16":           # block-scaled copies replace the bf16 experts
            E, F, D = dims.E, dims.F, dims.D
            U8 = dict(dtype=torch.uint8, device="cuda")
            cpb = 1 if experts == "mxfp8" else 2          # codes per byte
            self.mx = (torch.empty((E, 2 * F, D // cpb), **U8),
                       torch.empty((E, 2 * F, D // 32), **U8),
                       torch.empty((E, D, F // cpb), **U8), torch.empty((E, D, F // 32), **U8))
            quant = getattr(B, f"beam_{experts}_quantize")
            quant(w13, E * 2 * F, D, self.mx[0], self.mx[1])
            quant(w2, E * D, F, self.mx[2], self.mx[3])
            torch.cuda.synchronize()
            B.beam_check()
            del self.t["w13"], self.t["w2"], w13, w2
        K, V, ks, vs = synth.torch_kv_prior(dims, 1, ctx, kv, seed, layer)
        ct = torch.int16 if kv == "bf16" else torch.uint8
        self.K = torch.empty((1, dims.Hkv, Lmax, dims.d), dtype=ct, device="cuda")
        self.V = torch.empty((1, dims.Hkv, dims.d, Lmax), dtype=ct, device="cuda")
        self.K[:, :, :ctx] = K
        self.V[:, :, :, :ctx] = V.transpose(2, 3)
        del K, V
        self.ks, self.vs = ks, vs
        self.kv = B.kv_struct(self.K, self.V,
                              B.BEAM_KV_BF16 if kv == "bf16" else B.BEAM_KV_FP8_E4M3,
                              ks, vs, 1, Lmax)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: the layer runs on one GPU only (asked for {a.gpus}); "
              "sharding the layer across GPUs is not implemented.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import moe_decoder_layer_amd as B
    import synth

    torch.cuda.set_device(0)
    if a.copy_calibration:
        n = 1 << 28                                    # 1 GiB of fp32
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                          "launches": 5}))
        return

    if a.counters_prefill:
        prefill_leg(a, counters=True)
        return
    if a.counters_mx:
        mx_prefill_leg(a, only=a.counters_mx)
        return
    swa = decode_leg(a, 1)
    if a.counters or a.counters_step:
        return
    sets, dims, ex = swa.pop("_sets"), swa.pop("_dims"), swa.pop("_ex")
    us_step = swa["us_mean"]
    D = dims.D
    s = torch.cuda.current_stream()

    # --- dominant kernel: the selected-expert gate/up GEMV with SwiGLU ---------
    I16 = dict(dtype=torch.int16, device="cuda")
    x2, idx = swa.pop("_x2"), swa.pop("_idx")
    act = torch.empty((1, dims.topk + 1, dims.F), **I16)
    up_reps = 40
    stream = torch.cuda.Stream()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g2, stream=stream):
            for i in range(up_reps):
                B.beam_moe_experts_up(dims, 1, x2, idx, sets[i % 2].t["w13"], None, act)
    torch.cuda.synchronize()
    g2.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(5):
        g2.replay()
    e1.record(s)
    torch.cuda.synchronize()
    up_us = e0.elapsed_time(e1) * 1000.0 / (5 * up_reps)
    up_bytes = up_bytes_of(dims)
    up_gbs = up_bytes / (up_us * 1e-6) / 1e9
    step_bytes = swa["bytes_per_step"]
    step_gbs = step_bytes / (us_step * 1e-6) / 1e9
    log(f"[bench] expert gate/up GEMV: {up_us:.2f} us/launch, {up_gbs:.0f} GB/s; "
        f"step {step_gbs:.0f} GB/s over {step_bytes} B")
    del g2
    ceiling = hbm_read_ceiling()
    log(f"[bench] streaming-read ceiling (plain read kernel, 2 x 4 GiB): {ceiling:.0f} GB/s")

    out = {
        "metric": "Beam layer decode µs/step (b=1, 100K ctx) + prefill tok/s; % HBM/MFMA roofline",
        "value": round(us_step, 3),
        "unit": "µs/step",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(us_step / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "beam_swa_moe_layer_decode", "batch": 1, "context": ex["pos"],
                   "kv_cache": "bf16", "hidden": D, "q_heads": dims.Hq, "kv_heads": dims.Hkv,
                   "head_dim": dims.d, "window": dims.window, "experts": dims.E,
                   "topk": dims.topk, "expert_dff": dims.F, "weight_sets": 2,
                   "graph_chain": swa["graph_chain"]},
        "graph_replays": swa["graph_replays"],
        "us_per_step_distribution": swa["distribution"],
        "us_per_step_median": swa["us_median"],
        "us_per_step_p90": swa["us_p90"],
        "roofline": {"bound": "hbm", "kernel": "expert_w13_swiglu_kernel",
                     "achieved": round(up_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(up_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": up_bytes, "us_per_launch": round(up_us, 3)},
        "step_roofline": {"bound": "hbm", "bytes_per_step": step_bytes,
                          "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                          "measured_read_ceiling_gbs": round(ceiling, 1)},
    }
    cpu = {}
    if not a.no_cpu_baseline:
        cpu["decode_swa"] = cpu_decode(sets[0], dims, ex, "swa", a.cpu_steps)
    del sets
    torch.cuda.empty_cache()
    if not a.no_nope:
        nope = decode_leg(a, 2)
        nsets, ndims, nex = nope.pop("_sets"), nope.pop("_dims"), nope.pop("_ex")
        for k in ("_x2", "_idx"):
            nope.pop(k)
        out["decode_nope"] = nope
        if not a.no_cpu_baseline:
            cpu["decode_nope_fp8"] = cpu_decode(nsets[0], ndims, nex, "nope",
                                                max(2, a.cpu_steps // 2))
        del nsets
        torch.cuda.empty_cache()
    for fmt in ([] if a.no_mx else ["mxfp8", "mxfp4"]):
        mxr = decode_leg(a, 1, fmt)
        msets, x2m, idxm = mxr.pop("_sets"), mxr.pop("_x2"), mxr.pop("_idx")
        for k in ("_dims", "_ex"):
            mxr.pop(k)
        # the two block-scaled expert kernels alone, alternating weight sets
        wm = torch.full((1, dims.topk), 0.125, dtype=torch.float32, device="cuda")
        ym = torch.empty((1, D), **I16)
        wsm = torch.zeros(B.beam_workspace_size(dims, B.BEAM_OP_MOE, 1), dtype=torch.uint8,
                          device="cuda")
        call = getattr(B, f"beam_moe_swiglu_combine_{fmt}")
        moe_us = graph_us(lambda i: call(dims, 1, x2m, idxm, wm, *msets[i % 2].mx, ym, wsm), 40)
        moe_bytes = dims.topk * 3 * dims.F * D * EXPERT_BYTES_PER_32[fmt] // 32
        moe_gbs = moe_bytes / (moe_us * 1e-6) / 1e9
        log(f"[bench] {fmt} expert kernels: {moe_us:.2f} us per call, {moe_gbs:.0f} GB/s")
        mxr["experts_call"] = {"us": round(moe_us, 3), "bytes": moe_bytes,
                               "achieved_gbs": round(moe_gbs, 1),
                               "frac": round(moe_gbs / HBM_PEAK_GBS, 4)}
        out[f"decode_swa_{fmt}_experts"] = mxr
        del msets
        torch.cuda.empty_cache()
    if not a.no_1m:
        # the NoPE fp8 layer at a 2^20-token context: 2 GiB of fp8 KV per layer
        r1m = decode_leg(a, 2, ctx=1 << 20)
        for k in ("_sets", "_dims", "_ex", "_x2", "_idx"):
            r1m.pop(k)
        out["decode_nope_fp8_1m"] = r1m
        torch.cuda.empty_cache()
    if not a.no_head:
        out["lm_head_softcap_b1"] = head_leg()
        torch.cuda.empty_cache()
    if not a.no_stack:
        out["decode_stack_52"] = stack_leg(a)
        torch.cuda.empty_cache()
    if not a.no_flint:
        out["decode_flint_b128"] = {m: flint_leg(a, m) for m in ("swa", "nope")}
        torch.cuda.empty_cache()
    if not a.no_prefill:
        out["prefill"] = prefill_leg(a, cpu=cpu if not a.no_cpu_baseline else None)
        torch.cuda.empty_cache()
    if not a.no_mx_prefill:
        out["prefill_moe_mx"] = mx_prefill_leg(a)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_summary(cpu)
    print(json.dumps(out))


# bytes per 32 expert weights: bf16; e4m3 codes + one scale; e2m1 codes + one scale
EXPERT_BYTES_PER_32 = {"bf16": 64, "mxfp8": 33, "mxfp4": 17}


def head_leg():
    """The output head with the logit soft cap at one decode token: Beam's
    hidden size, a synthetic 131,072-entry vocabulary (the pages give none),
    two weight copies alternated so every call streams its 1.34 GB from HBM."""
    import torch

    import moe_decoder_layer_amd as B
    import synth
    D, V = 5120, 131072
    ws = [synth.torch_normal_bf16((V, D), 0.02, s, "head_w") for s in (0, 1)]
    x = synth.torch_normal_bf16((1, D), 1.0, 0, "head_x")
    logits = torch.empty((1, V), dtype=torch.float32, device="cuda")
    B.beam_lm_head_softcap(1, D, V, x, ws[0], 30.0, logits)
    torch.cuda.synchronize()
    B.beam_check()
    us = graph_us(lambda i: B.beam_lm_head_softcap(1, D, V, x, ws[i % 2], 30.0, logits), 20)
    nbytes = V * D * 2 + D * 2 + V * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"[bench] lm head + softcap (D {D}, V {V}, b 1): {us:.2f} us, {gbs:.0f} GB/s")
    return {"workload": "lm_head_softcap_decode", "hidden": D, "vocab": V, "cap": 30.0,
            "us": round(us, 3), "bytes": nbytes, "achieved_gbs": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def stack_leg(a):
    """One decode token through the whole Beam model on one GPU: the 52 layers
    in the model's schedule (beam_layer_kind: 43 sliding-window layers on
    512-slot ring caches, 9 NoPE layers on full caches, the token at position
    2^20, fp8 KV throughout; layers 0-2 dense) in one beam_decode_stack call,
    then the output head with the soft cap, one HIP graph per step. One GPU
    cannot hold 49 layers of bf16 experts (about 20 GB each), so the MoE layers
    take their weights from two sets used by alternate layers, and the dense
    layers likewise (a layer's selected experts, ~0.6 GB, evict the other set
    from the caches, so every layer still streams its weights from HBM); every
    layer has its own KV cache (18 GiB for the nine NoPE layers)."""
    import numpy as np
    import torch

    import moe_decoder_layer_amd as B
    import synth
    t0 = time.time()
    dims = synth.config(1).dims
    D, Fd, NL, ctx, V = dims.D, dims.Fd, 52, 1 << 20, 131072
    kinds = [B.beam_layer_kind(l, NL) for l in range(NL)]
    msets = [LayerSet(dims, seed, 200 + seed, 64, 64, "fp8") for seed in (0, 1)]
    dsets = [(synth.torch_normal_bf16((2 * Fd, D), 0.02, seed, "stack_dense_w13"),
              synth.torch_normal_bf16((D, Fd), 0.02, seed, "stack_dense_w2")) for seed in (0, 1)]
    U8 = dict(dtype=torch.uint8, device="cuda")
    npos = ctx + 64                   # positions [0, 2^20] (the token sits at 2^20)
    caches, kvs = [], []
    for l, (mode, dense) in enumerate(kinds):
        slots = 512 if mode == B.BEAM_SWA_ROPE else npos
        fill = 512 if mode == B.BEAM_SWA_ROPE else ctx
        Kp, Vp, ks, vs = synth.torch_kv_prior(dims, 1, fill, "fp8", 300, l)
        K = torch.empty((1, dims.Hkv, slots, dims.d), **U8)
        Vt = torch.empty((1, dims.Hkv, dims.d, slots), **U8)
        K[:, :, :fill] = Kp
        Vt[:, :, :, :fill] = Vp.transpose(2, 3)
        del Kp, Vp
        caches.append((K, Vt))
        kvs.append(B.kv_struct(K, Vt, B.BEAM_KV_FP8_E4M3, ks, vs, 1, slots,
                               npos if mode == B.BEAM_SWA_ROPE else 0))
    rope_h = np.zeros((npos, dims.d), np.float32)
    B.beam_rope_table(rope_h, npos, dims.d, dims.theta)
    rope = torch.from_numpy(rope_h).cuda()
    del rope_h
    layers = []
    for l, (mode, dense) in enumerate(kinds):
        w = dict(msets[l % 2].t)
        if dense:
            w["w13"], w["w2"] = dsets[l % 2]
        layers.append(B.stack_layer(mode, dense, w, kvs[l]))
    w_final = msets[0].t["w_next_pre"]
    w_head = synth.torch_normal_bf16((V, D), 0.02, 0, "stack_head_w")
    I16 = dict(dtype=torch.int16, device="cuda")
    h = synth.torch_normal_bf16((1, D), 1.0, 0, "stack_h")
    x = torch.empty((1, D), **I16)
    logits = torch.empty((1, V), dtype=torch.float32, device="cuda")
    pos = torch.tensor([ctx], dtype=torch.int32, device="cuda")
    seq = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(B.beam_decode_stack_workspace(dims, Fd, ctx + 1), **U8)
    log(f"[bench] 52-layer stack: weights, caches and RoPE table set up in "
        f"{time.time() - t0:.1f}s ({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")

    def step(k):
        B.beam_decode_stack(dims, Fd, 0, layers, w_final, h, x, pos, seq, rope, ctx, ws)
        B.beam_lm_head_softcap(1, D, V, x, w_head, 30.0, logits)

    step(0)                              # one eager step validates the composition
    torch.cuda.synchronize()
    B.beam_check()
    assert torch.isfinite(logits).all(), "non-finite logits"
    warm = max(1, min(a.warmup, 3))
    us, per, reps, _, dsrc = timed_steps(step, 1, warm, a.stack_steps, 1)
    B.beam_check()
    # algorithmic bytes: weights each layer reads, KV read and written, the head
    attn_w = dims.qkvg_rows * D * 2 + D * dims.Hq * dims.d * 2
    kv_tok = dims.Hkv * dims.d * 2          # K and V bytes of one position (fp8)
    nbytes = V * D * 2
    for mode, dense in kinds:
        nbytes += attn_w + kv_tok
        nbytes += (dims.window if mode == B.BEAM_SWA_ROPE else ctx + 1) * kv_tok
        nbytes += 3 * Fd * D * 2 if dense else dims.E * D * 4 + dims.topk * 3 * dims.F * D * 2
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"[bench] 52-layer decode step + head at 2^20 context: {us / 1000:.3f} ms/token "
        f"(median {np.median(per) / 1000:.3f}, p90 {np.percentile(per, 90) / 1000:.3f} over "
        f"{dsrc}), {1e6 / us:.1f} tok/s, {gbs:.0f} GB/s")
    res = {"workload": "beam_52_layer_decode_step", "layers": NL, "sliding_window_layers":
           sum(m == B.BEAM_SWA_ROPE for m, _ in kinds), "dense_layers": sum(d for _, d in kinds),
           "context": ctx, "kv_cache": "fp8", "sliding_window_cache": "ring of 512 slots",
           "experts": "bf16", "moe_weight_sets": 2, "lm_head_vocab": V, "steps": a.stack_steps,
           "warmup": warm, "graph_replays": reps, "distribution": dsrc,
           "ms_per_token": round(us / 1000, 4), "ms_median": round(float(np.median(per)) / 1000, 4),
           "ms_p90": round(float(np.percentile(per, 90)) / 1000, 4),
           "tokens_per_s": round(1e6 / us, 2), "bytes_per_step": nbytes,
           "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    del layers, kvs, caches, msets, dsets, rope, w_head
    return res


def graph_us(fn, reps):
    """Mean µs of one fn(i) call: reps calls captured in one HIP graph, the
    graph replayed five times between two events on the current stream."""
    import torch
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(reps):
                fn(i)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(5):
        g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / (5 * reps)


def timed_steps(step, nsets, warmup, steps, chain, min_replays=16):
    """Exactly `warmup` untimed steps, then exactly `steps` timed steps, of
    step(k) for absolute step index k (step k runs on weight set k % nsets).
    Steps are replayed from HIP graphs of `chain` steps (the last replay of a
    region holds the remainder); a graph is captured per (first weight set,
    length) so the alternation holds across replay boundaries. The per-step
    distribution (median, p90) comes from the timed replays when there are
    at least min_replays of them, else from min_replays further replays of
    the chain after the timed region (one graph replay costs a launch gap
    of several us, so a one-step chain would measure launches, not steps).
    Returns (us per step over the timed region, per-replay us-per-step of the
    distribution sample, timed replays, chain, distribution source)."""
    import numpy as np
    import torch
    c = max(1, min(chain, steps))
    graphs = {}

    def graph(k, n):
        key = (k % nsets, n)
        if key not in graphs:
            stream = torch.cuda.Stream()
            stream.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=stream):
                    for i in range(n):
                        step(k + i)
            torch.cuda.current_stream().wait_stream(stream)
            torch.cuda.synchronize()
            graphs[key] = g
        return graphs[key]

    def plan(k0, total):
        out, k = [], k0
        while k < k0 + total:
            n = min(c, k0 + total - k)
            out.append((k, n))
            k += n
        return out

    def replay(pl):
        s = torch.cuda.current_stream()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(pl) + 1)]
        evs[0].record(s)
        for r, (k, n) in enumerate(pl):
            graph(k, n).replay()
            evs[r + 1].record(s)
        torch.cuda.synchronize()
        per = np.array([evs[r].elapsed_time(evs[r + 1]) * 1000.0 / n
                        for r, (k, n) in enumerate(pl)])
        return evs[0].elapsed_time(evs[-1]) * 1000.0, per

    warm, timed = plan(0, warmup), plan(warmup, steps)
    for k, n in warm + timed:           # capture everything before any timing
        graph(k, n)
    for k, n in warm:
        graph(k, n).replay()
    torch.cuda.synchronize()
    total_us, per = replay(timed)
    us = total_us / steps
    source = "timed region"
    if len(timed) < min_replays:
        k0 = warmup + steps
        dist = [(k0 + i * c, c) for i in range(min_replays)]
        for k, n in dist:
            graph(k, n)
        _, per = replay(dist)
        source = f"{min_replays} replays of {c} steps after the timed region"
    del graphs
    return us, per, len(timed), c, source


def decode_leg(a, ci, experts="bf16", ctx=None):
    """Batch-1 decode layer-steps of config ci (1: SWA layer 10 on a 100K bf16
    cache; 2: NoPE layer 11 on a 100K fp8 cache), chained 8 per HIP graph over
    two alternating full weight sets. Each graph replay is timed on its own
    (HIP events between replays) for the mean, median and p90 per step.
    experts "mxfp8" / "mxfp4": the routed experts run from block-scaled copies.
    ctx: prior tokens in place of the config's (the cache grows to fit)."""
    import numpy as np
    import torch

    import moe_decoder_layer_amd as B
    import synth
    cfg = synth.config(ci)
    dims, ex = cfg.dims, cfg.extra
    pos0, Lmax, n, mode, kvt = ex["pos"], ex["Lmax"], ex["n"], ex["mode"], ex["kv"]
    if ctx is not None:
        pos0, Lmax = ctx, (ctx + 64) // 64 * 64
    t0 = time.time()
    sets = [LayerSet(dims, seed, ex["layer"], pos0, Lmax, kvt, experts) for seed in (0, 1)]
    log(f"[bench] {mode} decode ({experts} experts): weights + caches drawn in {time.time() - t0:.1f}s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")
    I16 = dict(dtype=torch.int16, device="cuda")
    D = dims.D
    h = synth.torch_normal_bf16((1, D), 1.0, 0, "bench_h")
    x = torch.empty((1, D), **I16)
    q = torch.empty((1, dims.Hq, dims.d), **I16)
    g = torch.empty((1, dims.G), **I16)
    o = torch.empty((1, dims.Hq, dims.d), **I16)
    y = torch.empty((1, D), **I16)
    x2 = torch.empty((1, D), **I16)
    y2 = torch.empty((1, D), **I16)
    idx = torch.empty((1, dims.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((1, dims.topk), dtype=torch.float32, device="cuda")
    pos = torch.tensor([pos0], dtype=torch.int32, device="cuda")
    seq = torch.zeros(1, dtype=torch.int32, device="cuda")
    rope = None
    if mode == "swa":
        rope_h = np.zeros((Lmax, dims.d), np.float32)
        B.beam_rope_table(rope_h, Lmax, dims.d, dims.theta)
        rope = torch.from_numpy(rope_h).cuda()
    attn_op = B.BEAM_OP_ATTN_SWA if mode == "swa" else B.BEAM_OP_ATTN_NOPE
    attn = B.beam_attn_swa if mode == "swa" else B.beam_attn_nope_ssmax
    m = B.BEAM_SWA_ROPE if mode == "swa" else B.BEAM_NOPE_SSMAX
    wsz = lambda op, ctx=0: torch.zeros(max(256, B.beam_workspace_size(dims, op, 1, ctx)),  # noqa
                                        dtype=torch.uint8, device="cuda")
    ws_qkv, ws_attn = wsz(B.BEAM_OP_QKV), wsz(attn_op, pos0 + 1)
    ws_fa = wsz(B.BEAM_OP_ATTN_DECODE_FUSED, pos0 + 1) if not a.unfused else None
    ws_r, ws_moe = wsz(B.BEAM_OP_ROUTER), wsz(B.BEAM_OP_MOE)
    moe_mx = getattr(B, f"beam_moe_swiglu_combine_{experts}", None)
    z = torch.empty((1, dims.Hq * dims.d), **I16)

    def step(L: LayerSet):
        t = L.t
        if a.unfused:
            B.beam_qk_norm_rope_ssmax_kvwrite(dims, 1, x, t["w_qkvg"], t["w_qnorm"], t["w_knorm"],
                                              pos, seq, m, rope, q, g, L.kv, ws_qkv)
            attn(dims, 1, q, pos, seq, L.kv, None, o, pos0, ws_attn)
            B.beam_out_gate(dims, 1, o, g, t["b_gate"], t["w_o"], y)
        else:  # projection + q/k epilogue + attention + gate, then o_proj alone
            B.beam_attn_decode_fused(dims, 1, x, t["w_qkvg"], t["w_qnorm"], t["w_knorm"], pos,
                                     seq, m, rope, L.kv, None, t["b_gate"], None, z, pos0, ws_fa)
            B.beam_out_gate(dims, 1, z, None, None, t["w_o"], y)
        # attention-side boundary + router in one call (the two calls fused)
        B.beam_boundary_router_fp32_grouped_topk(dims, 1, y, t["w_attn_post"], h, t["w_ffn_pre"],
                                                 x2, n, t["w_r"], t["b_corr"], idx, w, None,
                                                 ws_r)
        if experts != "bf16":
            moe_mx(dims, 1, x2, idx, w, *L.mx, y2, ws_moe)
        else:
            B.beam_moe_swiglu_combine(dims, 1, x2, idx, w, t["w13"], t["w2"], None, None, y2,
                                      ws_moe)
        B.beam_boundary_norm_residual(dims, 1, y2, t["w_ffn_post"], h, t["w_next_pre"], x, n + 1)

    # layer entry pre-norm once; then validate one eager chain
    B.beam_boundary_norm_residual(dims, 1, None, None, h, sets[0].t["w_attn_pre"], x, 0)
    if a.counters:
        step(sets[0])           # a routed token: x2 and idx as in a layer step
        act = torch.empty((1, dims.topk + 1, dims.F), **I16)
        torch.cuda.synchronize()
        for i in range(20):
            B.beam_moe_experts_up(dims, 1, x2, idx, sets[i % 2].t["w13"], None, act)
        torch.cuda.synchronize()
        B.beam_check()
        print(json.dumps({"counters_run": "expert_w13_swiglu_kernel", "launches": 20,
                          "algorithmic_bytes_per_launch": up_bytes_of(dims)}))
        return {}
    if a.counters_step:
        torch.cuda.synchronize()
        for i in range(8):
            step(sets[i % 2])
        torch.cuda.synchronize()
        B.beam_check()
        print(json.dumps({"counters_run": f"{mode} decode layer-steps", "steps": 8}))
        return {}
    # one eager chain validates the step before anything is captured
    for i in range(a.chain):
        step(sets[i % 2])
    B.beam_check()
    assert torch.isfinite(h.view(torch.bfloat16).float()).all(), "non-finite residual stream"
    steps = a.steps
    us_step, per, reps, chain, dsrc = timed_steps(lambda k: step(sets[k % 2]), 2, a.warmup,
                                                  steps, a.chain)
    B.beam_check()
    log(f"[bench] {mode} decode: {steps} layer-steps ({reps} graph replays of <= {chain}) in "
        f"{us_step * steps / 1000:.2f} ms: {us_step:.2f} us/step "
        f"(median {np.median(per):.2f}, p90 {np.percentile(per, 90):.2f} over {dsrc})")
    kv_read = dims.window if mode == "swa" else pos0 + 1
    kv_bytes = kv_read * dims.Hkv * dims.d * 2 * (2 if kvt == "bf16" else 1)
    kv_write = dims.Hkv * dims.d * 2 * (2 if kvt == "bf16" else 1)
    expert_bytes = dims.topk * 3 * dims.F * D * EXPERT_BYTES_PER_32[experts] // 32
    step_bytes = (dims.qkvg_rows * D * 2 + D * dims.Hq * dims.d * 2 + dims.E * D * 4
                  + expert_bytes + kv_bytes + kv_write)
    res = {"workload": f"beam_{mode}_moe_layer_decode", "kv_cache": kvt, "experts": experts,
           "context": pos0, "attention_call": "separate" if a.unfused else "fused",
           "steps": steps, "warmup": a.warmup, "validation_steps": a.chain,
           "graph_replays": reps, "graph_chain": chain, "distribution": dsrc,
           "us_mean": round(us_step, 3), "us_median": round(float(np.median(per)), 3),
           "us_p90": round(float(np.percentile(per, 90)), 3), "bytes_per_step": step_bytes,
           "hbm_frac": round(step_bytes / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "_sets": sets, "_dims": dims, "_ex": ex, "_x2": x2, "_idx": idx}
    return res


class FlintSet:
    """The second model's layer (pre-norm, sinks, no gate, top-6 + shared
    expert) with a batch of S sequences' bf16 caches, random-init, seeded."""

    def __init__(self, dims, seed, layer, S, ctx, Lmax):
        import numpy as np
        import torch

        import moe_decoder_layer_amd as B
        import synth
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(  # noqa: E731
            a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
        p = synth.make_params(dims, seed, layer, experts=False, projections=False)
        self.t = {k: dev(v) for k, v in p.items()}
        nb = lambda shape, *key: synth.torch_normal_bf16(shape, 0.02, seed, layer, *key)  # noqa
        self.t["w_qkvg"] = nb((dims.qkvg_rows, dims.D), "w_qkvg")
        self.t["w_o"] = nb((dims.D, dims.Hq * dims.d), "w_o")
        w13 = torch.empty((dims.E, 2 * dims.F, dims.D), dtype=torch.int16, device="cuda")
        w2 = torch.empty((dims.E, dims.D, dims.F), dtype=torch.int16, device="cuda")
        for e in range(dims.E):
            synth.torch_normal_bf16((2 * dims.F, dims.D), 0.02, seed, layer, "w13", e, out=w13[e])
            synth.torch_normal_bf16((dims.D, dims.F), 0.02, seed, layer, "w2", e, out=w2[e])
        self.t["w13"], self.t["w2"] = w13, w2
        self.t["shared_w13"] = nb((2 * dims.F, dims.D), "w13", "shared")
        self.t["shared_w2"] = nb((dims.D, dims.F), "w2", "shared")
        K, V, ks, vs = synth.torch_kv_prior(dims, S, ctx, "bf16", seed, layer)
        self.K = torch.empty((S, dims.Hkv, Lmax, dims.d), dtype=torch.int16, device="cuda")
        self.V = torch.empty((S, dims.Hkv, dims.d, Lmax), dtype=torch.int16, device="cuda")
        self.K[:, :, :ctx] = K
        self.V[:, :, :, :ctx] = V.transpose(2, 3)
        del K, V
        self.kv = B.kv_struct(self.K, self.V, B.BEAM_KV_BF16, ks, vs, S, Lmax)


def flint_leg(a, mode):
    """The second model's layer shape as a batch of decode steps: 128
    sequences, one new token each at position 8,192 of a bf16 cache (SWA: the
    last 513 keys; NoPE: all 8,193), pre-norm layer with per-head sinks, no
    output gate, sigmoid top-6 of 256 experts plus a shared expert. Steps are
    chained over two alternating weight sets in one HIP graph, as the Beam
    legs. Bytes per step count each distinct routed expert once (the
    selected experts of a step are read once whatever number of tokens
    chose them)."""
    import numpy as np
    import torch

    import moe_decoder_layer_amd as B
    import synth
    cfg = synth.config(4)
    dims, ex = cfg.dims, cfg.extra
    S, ctx, Lmax = ex["B"], ex["ctx"], ex["Lmax"]
    T, D = S, dims.D
    layer = 3
    t0 = time.time()
    sets = [FlintSet(dims, seed, layer, S, ctx, Lmax) for seed in (0, 1)]
    log(f"[bench] flint {mode} b{S} decode: weights + caches drawn in {time.time() - t0:.1f}s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")
    I16 = dict(dtype=torch.int16, device="cuda")
    h = synth.torch_normal_bf16((T, D), 1.0, 0, "bench_flint_h")
    x = torch.empty((T, D), **I16)
    q = torch.empty((T, dims.Hq, dims.d), **I16)
    o = torch.empty((T, dims.Hq, dims.d), **I16)
    y = torch.empty((T, D), **I16)
    x2 = torch.empty((T, D), **I16)
    y2 = torch.empty((T, D), **I16)
    idx = torch.empty((T, dims.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, dims.topk), dtype=torch.float32, device="cuda")
    pos = torch.full((T,), ctx, dtype=torch.int32, device="cuda")
    seq = torch.arange(T, dtype=torch.int32, device="cuda")
    rope = None
    if mode == "swa":
        rope_h = np.zeros((Lmax, dims.d), np.float32)
        B.beam_rope_table(rope_h, Lmax, dims.d, dims.theta)
        rope = torch.from_numpy(rope_h).cuda()
    attn_op = B.BEAM_OP_ATTN_SWA if mode == "swa" else B.BEAM_OP_ATTN_NOPE
    attn = B.beam_attn_swa if mode == "swa" else B.beam_attn_nope_ssmax
    m = B.BEAM_SWA_ROPE if mode == "swa" else B.BEAM_NOPE_SSMAX
    wsz = lambda op, ctx_=0: torch.zeros(max(256, B.beam_workspace_size(dims, op, T, ctx_)),  # noqa
                                         dtype=torch.uint8, device="cuda")
    ws_qkv, ws_attn, ws_og = wsz(B.BEAM_OP_QKV), wsz(attn_op, ctx + 1), wsz(B.BEAM_OP_OUT_GATE)
    ws_r, ws_moe = wsz(B.BEAM_OP_ROUTER), wsz(B.BEAM_OP_MOE)

    def step(L: FlintSet):
        t = L.t
        B.beam_qk_norm_rope_ssmax_kvwrite(dims, T, x, t["w_qkvg"], t["w_qnorm"], t["w_knorm"],
                                          pos, seq, m, rope, q, None, L.kv, ws_qkv)
        attn(dims, T, q, pos, seq, L.kv, t["sink"], o, ctx, ws_attn)
        B.beam_out_gate(dims, T, o, None, None, t["w_o"], y, ws_og)
        B.beam_boundary_norm_residual(dims, T, y, None, h, t["w_ffn_pre"], x2, 0)
        B.beam_router_fp32_grouped_topk(dims, T, x2, t["w_r"], t["b_corr"], idx, w, None, ws_r)
        B.beam_moe_swiglu_combine(dims, T, x2, idx, w, t["w13"], t["w2"], t["shared_w13"],
                                  t["shared_w2"], y2, ws_moe)
        B.beam_boundary_norm_residual(dims, T, y2, None, h, t["w_next_pre"], x, 0)

    B.beam_boundary_norm_residual(dims, T, None, None, h, sets[0].t["w_attn_pre"], x, 0)
    distinct = []
    for i in range(a.chain):
        step(sets[i % 2])
        distinct.append(len(np.unique(idx.cpu().numpy())))
    B.beam_check()
    assert torch.isfinite(h.view(torch.bfloat16).float()).all(), "non-finite residual stream"
    steps = min(a.steps, 80)
    us_step, per, reps, chain, _ = timed_steps(lambda k: step(sets[k % 2]), 2,
                                               min(a.warmup, 16), steps, a.chain)
    B.beam_check()
    ne = float(np.mean(distinct))
    keys = (dims.window if mode == "swa" else ctx + 1)
    kv_bytes = T * keys * dims.Hkv * dims.d * 2 * 2
    step_bytes = int(dims.qkvg_rows * D * 2 + D * dims.Hq * dims.d * 2 + dims.E * D * 4
                     + (ne + 1) * 3 * dims.F * D * 2 + kv_bytes + T * dims.Hkv * dims.d * 4)
    log(f"[bench] flint {mode} b{S} decode: {us_step:.2f} us/step (median {np.median(per):.2f}), "
        f"{ne:.1f} distinct experts/step, {step_bytes / (us_step * 1e-6) / 1e9:.0f} GB/s")
    del sets
    return {"workload": f"flint_{mode}_moe_layer_decode_b{S}", "batch": S, "context": ctx,
            "kv_cache": "bf16", "steps": steps, "warmup": min(a.warmup, 16),
            "graph_replays": reps, "us_mean": round(us_step, 3),
            "us_median": round(float(np.median(per)), 3),
            "tokens_per_s": round(T / (us_step * 1e-6), 1),
            "distinct_experts_per_step": round(ne, 1), "bytes_per_step": step_bytes,
            "hbm_frac": round(step_bytes / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def hbm_read_ceiling():
    """Read bandwidth of the library's plain streaming-read kernel over two
    alternating 4 GiB buffers: a measured ceiling beside the nominal 8 TB/s."""
    import torch

    import moe_decoder_layer_amd as B
    bufs = [torch.ones(1 << 30, dtype=torch.float32, device="cuda") for _ in range(2)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i in range(2):
        B.beam_hbm_read(bufs[i], sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(10):
        B.beam_hbm_read(bufs[i % 2], sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = 10 * bufs[0].numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del bufs
    return gbs


MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)


def up_bytes_of(dims):
    """Algorithmic HBM bytes of one expert gate/up launch at batch 1: the 8
    selected experts' gate and up rows, the activation row in, act out."""
    return dims.topk * 2 * dims.F * dims.D * 2 + dims.D * 2 + dims.topk * dims.F * 2


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expert_w13_swiglu_b1_traffic.md")
KERNEL_SRCS = [os.path.join(ROOT, "moe_decoder_layer_amd", "csrc", f)
               for f in ("k_gemv.hip", "common.h")]


def kernel_source_hash():
    """sha256 over the sources the expert gate/up kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the expert gate/up kernel from the committed
    rocprofv3 counter summary, or None when that summary is missing or was
    taken on a different version of the kernel source."""
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = {}
    for line in txt.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    try:
        src_hash = kernel_source_hash()
    except OSError:
        return None
    if fields.get("kernel_source_sha256") != src_hash:
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def prefill_leg(a, cpu=None, counters=False):
    """Chunked prefill: 8 sequences x 2048 new tokens, each after 100,000 prior
    tokens (bf16 cache), through one NoPE MoE layer, one SWA MoE layer and the
    dense layer 0. Returns per-layer ms, tok/s and MFMA-roofline fraction.
    cpu: a dict that gets the CPU oracle's sample of the NoPE layer.
    counters: one eager pass of each layer only (for rocprofv3 --pmc)."""
    import numpy as np
    import torch

    import moe_decoder_layer_amd as B
    import synth
    cfg = synth.config(3)
    ex = cfg.extra
    S, C, prior, Lmax = ex["S"], ex["chunk"], ex["prior"], ex["Lmax"]
    T = S * C
    base = synth.config(1).dims
    I16 = dict(dtype=torch.int16, device="cuda")
    pos = torch.tensor(np.concatenate([np.arange(prior, prior + C)] * S), dtype=torch.int32,
                       device="cuda")
    seq = torch.tensor(np.repeat(np.arange(S), C), dtype=torch.int32, device="cuda")
    rope_h = np.zeros((Lmax, base.d), np.float32)
    B.beam_rope_table(rope_h, Lmax, base.d, base.theta)
    rope = torch.from_numpy(rope_h).cuda()
    res = {}
    for name, layer in (("nope_moe", ex["layers"]["nope_moe"]), ("swa_moe", ex["layers"]["swa_moe"]),
                        ("dense", ex["layers"]["dense"])):
        dims = base
        mode = "swa" if name != "nope_moe" else "nope"
        ffn = "dense" if name == "dense" else "moe"
        n = 2 * layer + 1
        t0 = time.time()
        p = synth.make_params(dims, 0, layer, experts=False, projections=False)
        t = {k: torch.from_numpy(np.ascontiguousarray(v.view(np.int16) if v.dtype == np.uint16
                                                      else v)).cuda() for k, v in p.items()}
        t["w_qkvg"] = synth.torch_normal_bf16((dims.qkvg_rows, dims.D), 0.02, 0, layer, "w_qkvg")
        t["w_o"] = synth.torch_normal_bf16((dims.D, dims.Hq * dims.d), 0.02, 0, layer, "w_o")
        if ffn == "moe":
            w13 = torch.empty((dims.E, 2 * dims.F, dims.D), **I16)
            w2 = torch.empty((dims.E, dims.D, dims.F), **I16)
            for e in range(dims.E):
                synth.torch_normal_bf16((2 * dims.F, dims.D), 0.02, 0, layer, "w13", e, out=w13[e])
                synth.torch_normal_bf16((dims.D, dims.F), 0.02, 0, layer, "w2", e, out=w2[e])
        else:
            w13 = synth.torch_normal_bf16((2 * dims.Fd, dims.D), 0.02, 0, layer, "dense_w13")
            w2 = synth.torch_normal_bf16((dims.D, dims.Fd), 0.02, 0, layer, "dense_w2")
        K = torch.empty((S, dims.Hkv, Lmax, dims.d), **I16)
        V = torch.empty((S, dims.Hkv, dims.d, Lmax), **I16)
        Kp, Vp, _, _ = synth.torch_kv_prior(dims, S, prior, "bf16", 0, layer)
        K[:, :, :prior] = Kp
        V[:, :, :, :prior] = Vp.transpose(2, 3)
        del Kp, Vp
        kv = B.kv_struct(K, V, B.BEAM_KV_BF16, 1.0, 1.0, S, Lmax)
        h0 = synth.torch_normal_bf16((T, dims.D), 1.0, 0, "prefill_h", name)
        h = torch.empty_like(h0)
        x = torch.empty((T, dims.D), **I16)
        q = torch.empty((T, dims.Hq, dims.d), **I16)
        g = torch.empty((T, dims.G), **I16)
        o = torch.empty((T, dims.Hq, dims.d), **I16)
        y = torch.empty((T, dims.D), **I16)
        x2 = torch.empty((T, dims.D), **I16)
        y2 = torch.empty((T, dims.D), **I16)
        idx = torch.empty((T, dims.topk), dtype=torch.int32, device="cuda")
        w = torch.empty((T, dims.topk), dtype=torch.float32, device="cuda")
        wsz = lambda op, dd=dims: torch.zeros(  # noqa: E731
            max(256, B.beam_workspace_size(dd, op, T, prior + C)), dtype=torch.uint8, device="cuda")
        ws_q, ws_a, ws_o, ws_r = (wsz(B.BEAM_OP_QKV), wsz(B.BEAM_OP_ATTN_NOPE),
                                  wsz(B.BEAM_OP_OUT_GATE), wsz(B.BEAM_OP_ROUTER))
        if ffn == "moe":
            ws_f = wsz(B.BEAM_OP_MOE)
        else:
            ws_f = wsz(B.BEAM_OP_DENSE, synth.with_dims(synth.Config("", dims), F=dims.Fd).dims)
        attn = B.beam_attn_nope_ssmax if mode == "nope" else B.beam_attn_swa
        m = B.BEAM_NOPE_SSMAX if mode == "nope" else B.BEAM_SWA_ROPE
        log(f"[bench] prefill {name}: set up in {time.time() - t0:.1f}s")

        def layer_fwd():
            h.copy_(h0)
            B.beam_boundary_norm_residual(dims, T, None, None, h, t["w_attn_pre"], x, 0)
            B.beam_qk_norm_rope_ssmax_kvwrite(dims, T, x, t["w_qkvg"], t["w_qnorm"], t["w_knorm"],
                                              pos, seq, m, rope if mode == "swa" else None, q, g,
                                              kv, ws_q)
            attn(dims, T, q, pos, seq, kv, None, o, prior + C - 1, ws_a)
            B.beam_out_gate(dims, T, o, g, t["b_gate"], t["w_o"], y, ws_o)
            B.beam_boundary_norm_residual(dims, T, y, t["w_attn_post"], h, t["w_ffn_pre"], x2, n)
            if ffn == "moe":
                B.beam_router_fp32_grouped_topk(dims, T, x2, t["w_r"], t["b_corr"], idx, w, None,
                                                ws_r)
                B.beam_moe_swiglu_combine(dims, T, x2, idx, w, w13, w2, None, None, y2, ws_f)
            else:
                B.beam_dense_swiglu(T, dims.D, dims.Fd, x2, w13, w2, y2, ws_f)
            B.beam_boundary_norm_residual(dims, T, y2, t["w_ffn_post"], h, t["w_next_pre"], x,
                                          n + 1)

        layer_fwd()
        torch.cuda.synchronize()
        B.beam_check()
        if counters:
            log(f"[bench] prefill {name}: one pass for counters")
            del t, w13, w2, K, V, ws_f, ws_q, ws_a
            torch.cuda.empty_cache()
            continue
        reps = a.prefill_reps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            layer_fwd()
        e1.record()
        torch.cuda.synchronize()
        B.beam_check()
        ms = e0.elapsed_time(e1) / reps
        keys = (S * (C * prior + C * (C + 1) // 2)) if mode == "nope" else T * dims.window
        proj = 2 * dims.D * dims.qkvg_rows + 2 * dims.Hq * dims.d * dims.D
        ffn_fl = (dims.topk * 3 * 2 * dims.D * dims.F) if ffn == "moe" else 3 * 2 * dims.D * dims.Fd
        flops = T * (proj + ffn_fl) + keys * 4 * dims.d * dims.Hq
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 3), "tok_s": round(T / (ms * 1e-3), 1),
                     "algorithmic_flop": flops, "tflops": round(tf, 1),
                     "mfma_frac": round(tf / MFMA_PEAK_TFLOPS, 4)}
        log(f"[bench] prefill {name}: {ms:.2f} ms/layer, {T / ms * 1e3:.0f} tok/s, {tf:.0f} TFLOP/s")
        if cpu is not None and name == "nope_moe":
            cpu["prefill_nope_moe"] = cpu_prefill(t, w13, w2, K, V, h0, dims, mode, n, prior, 6)
            cpu["prefill_nope_moe"]["gpu_tok_s"] = res[name]["tok_s"]
        del t, w13, w2, K, V, ws_f, ws_q, ws_a
        torch.cuda.empty_cache()
    res["workload"] = "8 sequences x 2048 new tokens after 100,000 prior tokens each, bf16 cache"
    return res


FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak (published)


def mx_prefill_leg(a, only=None):
    """The routed-expert FFN of a prefill chunk alone (8 x 2048 tokens, the
    router's own top-8 choice over all 256 experts of random weights): the
    bf16 grouped GEMMs against the block-scaled ones (MXFP8 activations times
    MXFP8 or MXFP4 weights on the scaled matrix cores). Each variant's
    algorithmic flops (T * topk * 3 * 2 * D * F) per call, against the bf16
    peak for bf16 and the fp8 peak for the scaled variants (e2m1 weights with
    e4m3 activations run at the fp8 rate). only: run one variant once (for
    rocprofv3 --pmc)."""
    import numpy as np
    import torch

    import moe_decoder_layer_amd as B
    import synth
    dims = synth.config(1).dims
    T = 8 * 2048
    I16 = dict(dtype=torch.int16, device="cuda")
    U8 = dict(dtype=torch.uint8, device="cuda")
    t0 = time.time()
    p = synth.make_params(dims, 0, 4, experts=False, projections=False)
    w_r = torch.from_numpy(np.ascontiguousarray(p["w_r"])).cuda()
    b_corr = torch.from_numpy(np.ascontiguousarray(p["b_corr"])).cuda()
    x = synth.torch_normal_bf16((T, dims.D), 1.0, 0, "mx_prefill_x")
    idx = torch.empty((T, dims.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, dims.topk), dtype=torch.float32, device="cuda")
    ws = lambda op: torch.zeros(max(256, B.beam_workspace_size(dims, op, T)), **U8)  # noqa: E731
    B.beam_router_fp32_grouped_topk(dims, T, x, w_r, b_corr, idx, w, None, ws(B.BEAM_OP_ROUTER))
    E, F, D = dims.E, dims.F, dims.D
    w13 = torch.empty((E, 2 * F, D), **I16)
    w2 = torch.empty((E, D, F), **I16)
    for e in range(E):
        synth.torch_normal_bf16((2 * F, D), 0.02, 0, 4, "w13", e, out=w13[e])
        synth.torch_normal_bf16((D, F), 0.02, 0, 4, "w2", e, out=w2[e])
    y = torch.empty((T, D), **I16)
    variants = {}
    for fmt, wbits in (("mxfp8", 8), ("mxfp4", 4)):
        if only is not None and only != fmt:
            continue
        div = 1 if wbits == 8 else 2
        c13, s13 = torch.empty((E * 2 * F, D // div), **U8), torch.empty((E * 2 * F, D // 32), **U8)
        c2, s2 = torch.empty((E * D, F // div), **U8), torch.empty((E * D, F // 32), **U8)
        getattr(B, f"beam_{fmt}_quantize")(w13, E * 2 * F, D, c13, s13)
        getattr(B, f"beam_{fmt}_quantize")(w2, E * D, F, c2, s2)
        wsm = ws(B.BEAM_OP_MOE_MX_SCALED)
        variants[fmt] = (lambda wb=wbits, c13=c13, s13=s13, c2=c2, s2=s2, wsm=wsm:
                         B.beam_moe_swiglu_combine_mx_scaled(dims, T, x, idx, w, wb, c13, s13, c2,
                                                             s2, y, wsm))
    if only is None or only == "bf16":
        wsb = ws(B.BEAM_OP_MOE)
        variants["bf16"] = lambda: B.beam_moe_swiglu_combine(dims, T, x, idx, w, w13, w2, None,
                                                             None, y, wsb)
    torch.cuda.synchronize()
    B.beam_check()
    log(f"[bench] prefill MoE (block-scaled): set up in {time.time() - t0:.1f}s")
    flops = T * dims.topk * 3 * 2 * D * F
    res = {}
    for name, fn in variants.items():
        fn()
        torch.cuda.synchronize()
        B.beam_check()
        if only is not None:
            continue
        reps = max(3, a.prefill_reps * 2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        B.beam_check()
        ms = e0.elapsed_time(e1) / reps
        tf = flops / (ms * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS if name == "bf16" else FP8_PEAK_TFLOPS
        res[name] = {"ms": round(ms, 3), "tflops": round(tf, 1), "peak_tflops": peak,
                     "frac": round(tf / peak, 4)}
        log(f"[bench] prefill MoE {name}: {ms:.3f} ms, {tf:.0f} TFLOP/s ({tf / peak:.3f} of peak)")
    res["algorithmic_flop"] = flops
    res["workload"] = ("routed experts of 8 x 2048 prefill tokens, top-8 of 256 experts "
                       "(router on random weights), D 5120, F 2560")
    del w13, w2, variants
    return res


def _host_threads():
    """Threads the oracle's BLAS actually runs with, the CPU model and the
    process's CPU affinity."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    aff = sorted(os.sched_getaffinity(0))
    return int(threads), model, aff


class _Fetch:
    """Device -> host copies of expert weights, timed so that their time can
    be taken out of the oracle's (the copies are not oracle work)."""

    def __init__(self, w13, w2):
        self.w13, self.w2, self.s = w13, w2, 0.0

    def __call__(self, e):
        import numpy as np
        t0 = time.perf_counter()
        r = (self.w13[e].cpu().numpy().view(np.uint16), self.w2[e].cpu().numpy().view(np.uint16))
        self.s += time.perf_counter() - t0
        return r


def _host_params(t):
    import numpy as np
    import torch
    return {k: (v.cpu().numpy().view(np.uint16) if v.dtype == torch.int16 else v.cpu().numpy())
            for k, v in t.items() if k not in ("w13", "w2")}


def cpu_decode(L: "LayerSet", dims, ex, mode, nsteps):
    """The CPU oracle, untuned, on a bounded sample of a decode leg: nsteps
    chained layer-steps of the same workload (same weights; the same cache,
    copied to the host before the timer). The expert weights a step selects
    are copied from the device on demand and that copy time is excluded."""
    import numpy as np

    import synth
    from oracle import layer as OL
    from oracle.numerics import bf16_bits_to_f64, f64_to_bf16_bits
    P = _host_params(L.t)
    pos0 = ex["pos"]
    if mode == "swa":                     # the window is all a sliding-window step reads
        lo = pos0 - dims.window + 1
        cache = OL.KVCache.empty(1, dims.Hkv, pos0 + 1, dims.d)
        cache.K[:, :, lo:pos0] = bf16_bits_to_f64(L.K[:, :, lo:pos0].cpu().numpy().view(np.uint16))
        cache.V[:, :, lo:pos0] = bf16_bits_to_f64(
            L.V[:, :, :, lo:pos0].transpose(2, 3).contiguous().cpu().numpy().view(np.uint16))
    else:                                 # fp8 codes of the whole context
        cache = OL.KVCache.empty(1, dims.Hkv, pos0 + 1, dims.d, "fp8", L.ks, L.vs)
        cache.K[:, :, :pos0] = L.K[:, :, :pos0].cpu().numpy()
        cache.V[:, :, :pos0] = L.V[:, :, :, :pos0].transpose(2, 3).contiguous().cpu().numpy()
    fetch = _Fetch(L.t["w13"], L.t["w2"])
    h = synth.make_h((1, dims.D), 0, "cpu_baseline", mode)
    t0 = time.perf_counter()
    for _ in range(nsteps):
        r = OL.layer_forward(dims, P, h, [pos0], [0], cache, mode, ex["n"], get_expert=fetch)
        h = f64_to_bf16_bits(r["h_out"])
    dt = time.perf_counter() - t0 - fetch.s
    log(f"[bench] cpu oracle {mode} decode: {dt / nsteps * 1e3:.0f} ms/step over {nsteps} steps "
        f"({fetch.s:.1f}s of expert copies excluded)")
    return {"us_per_step": round(dt / nsteps * 1e6, 1), "steps": nsteps,
            "oracle_s": round(dt, 2), "expert_copy_s_excluded": round(fetch.s, 2),
            "workload": f"beam_{mode}_moe_layer_decode", "kv_cache": "bf16" if mode == "swa"
            else "fp8", "context": pos0}


def cpu_prefill(t, w13, w2, K, V, h0, dims, mode, n, prior, ntok):
    """The CPU oracle on a bounded sample of the prefill workload: the first
    ntok tokens of sequence 0's chunk (positions prior ..), attending over
    the same prior cache (copied to the host before the timer), through the
    same layer; reported as tokens per second."""
    import numpy as np

    from oracle import layer as OL
    from oracle.numerics import bf16_bits_to_f64
    P = _host_params(t)
    cache = OL.KVCache.empty(1, dims.Hkv, prior + ntok, dims.d)
    cache.K[:, :, :prior] = bf16_bits_to_f64(K[:1, :, :prior].cpu().numpy().view(np.uint16))
    cache.V[:, :, :prior] = bf16_bits_to_f64(
        V[:1, :, :, :prior].transpose(2, 3).contiguous().cpu().numpy().view(np.uint16))
    h = h0[:ntok].cpu().numpy().view(np.uint16)
    fetch = _Fetch(w13, w2)
    pos = np.arange(prior, prior + ntok)
    t0 = time.perf_counter()
    OL.layer_forward(dims, P, h, pos, np.zeros(ntok, int), cache, mode, n, get_expert=fetch)
    dt = time.perf_counter() - t0 - fetch.s
    log(f"[bench] cpu oracle {mode} prefill sample: {ntok} tokens in {dt:.1f}s "
        f"({fetch.s:.1f}s of expert copies excluded)")
    return {"tok_s": round(ntok / dt, 4), "tokens": ntok, "oracle_s": round(dt, 2),
            "expert_copy_s_excluded": round(fetch.s, 2),
            "workload": f"{ntok} tokens of one sequence's 2048-token chunk after {prior} prior "
                        f"tokens, {mode} MoE layer"}


def cpu_summary(cpu):
    """The cpu_baseline object: the headline decode leg's oracle time, with
    the other legs' samples beside it."""
    threads, model, aff = _host_threads()
    d = cpu.get("decode_swa", {})
    return {"value": d.get("us_per_step"), "unit": "µs/step", "cores": threads,
            "kind": "oracle",
            "sample": (f"{d.get('steps')} chained decode layer-steps of the same workload "
                       "(float64 NumPy oracle, cache window copied to the host before the "
                       "timer, the selected experts' device-to-host copies excluded); "
                       "further samples under legs"),
            "cpu_model": model, "affinity": f"{len(aff)} cpus ({aff[0]}-{aff[-1]})" if aff
            else "", "legs": cpu}


if __name__ == "__main__":
    main()
