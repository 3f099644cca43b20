"""The second model's layer form ("vLLM Day-0 support: Recursive's Flint",
Flint model architecture section): pre-norm with a plain residual, per-head
attention sinks, no output gate, sigmoid top-6 routing without groups plus a
shared expert, a 513-key window. Run as a batch of decode steps: every call
carries one new token for each of many sequences, each at its own position,
so attention runs split-K per token over that token's sequence (GPU)."""
import numpy as np
import pytest

import synth
from beamrun import Cache, Params, run_layer
from test_gpu_layer import check_end_to_end, check_stages

pytestmark = pytest.mark.gpu


def _flint(S, ctx, Lmax, kv, mode, E=64, seed=0, layer=3):
    cfg = synth.with_dims(synth.config(4), E=E)
    dims = cfg.dims
    P = Params(dims, seed, layer, moe=True)
    Kp, Vp, ks, vs = synth.torch_kv_prior(dims, S, ctx, kv, seed, layer)
    cache = Cache(dims, S, Lmax, kv, ks, vs)
    cache.fill_prior(Kp, Vp)
    # one token per sequence, positions spread over the prior (some windows
    # clipped at position 0, some tokens deep in their context)
    pos = (ctx - 1 - (np.arange(S) * 97) % ctx).astype(np.int32)
    seq = np.arange(S, dtype=np.int32)
    h = synth.make_h((S, dims.D), seed, "flint", mode, kv, S)
    return dims, P, cache, h, pos, seq


@pytest.mark.parametrize("S,ctx,Lmax,kv,mode", [
    (24, 900, 1024, "bf16", "swa"), (24, 900, 1024, "bf16", "nope"),
    (24, 900, 1024, "fp8", "swa"), (24, 900, 1024, "fp8", "nope"),
    # 128 sequences x 4 kv heads: more (token, kv head) pairs than the
    # last-workgroup merge has counters, so the merge kernel runs
    (128, 1200, 1280, "bf16", "swa"), (128, 1200, 1280, "fp8", "nope"),
])
def test_flint_batch_decode(S, ctx, Lmax, kv, mode):
    dims, P, cache, h, pos, seq = _flint(S, ctx, Lmax, kv, mode)
    ocache = cache.oracle()                     # prior only, before the layer writes
    g = run_layer(dims, P, cache, h, pos, seq, mode, 0, sandwich=False)
    check_stages(dims, P, cache, g, pos, seq, mode, 0, "moe", sink=P.np("sink"),
                 sandwich=False)
    check_end_to_end(dims, P, ocache, g, h, pos, seq, mode, 0, "moe", sandwich=False)
