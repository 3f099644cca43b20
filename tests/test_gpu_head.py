"""The output head with the logit soft cap (beam_lm_head_softcap) against the
oracle: fp32 logits within 1e-5 of the row's largest |z| (fp32 accumulation
over D) plus four binary32 ulps of the cap (the hardware tanh), on the
decode GEMV (T <= 4, and any T when D is not a multiple of 64) and on the
matrix-core GEMM with the cap applied in place (T > 4)."""
import numpy as np
import pytest
import torch

import moe_decoder_layer_amd as B
import synth
from beamrun import dev, host_bits
from oracle import layer as L
from oracle.numerics import bf16_bits_to_f64

pytestmark = pytest.mark.gpu


def _check(got, x, w_bits, cap):
    ref = L.lm_head_softcap(x, w_bits, cap)
    z = L.lm_head_softcap(x, w_bits, 0.0)
    tol = 1e-5 * np.abs(z).max(axis=1, keepdims=True) + 4 * 2.0 ** -24 * cap
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= tol), (err / tol).max()


@pytest.mark.parametrize("T,D,V", [(1, 256, 1000), (3, 256, 1000), (4, 256, 1000),
                                   (5, 256, 1000), (300, 256, 1000), (5, 200, 777),
                                   (1, 5120, 4099), (64, 5120, 4099)])
@pytest.mark.parametrize("cap", [30.0, 0.0])
def test_lm_head(T, D, V, cap):
    w = synth.normal_bf16((V, D), 0.02, 0, "head_w", D, V)
    x = synth.normal_bf16((T, D), 30.0, 0, "head_x", T, D)   # logits spread over the cap
    out = torch.empty((T, V), dtype=torch.float32, device="cuda")
    B.beam_lm_head_softcap(T, D, V, dev(x), dev(w), cap, out)
    B.beam_check()
    _check(out.cpu().numpy(), bf16_bits_to_f64(x), w, cap)


def test_lm_head_full_vocab_decode():
    """Beam's hidden size with a synthetic 131,072-entry vocabulary (the pages
    give none) at one decode token: 4,096 sampled vocabulary rows plus the
    first and last, checked against the oracle."""
    D, V, T = 5120, 131072, 1
    w = synth.torch_normal_bf16((V, D), 0.02, 0, "head_full")
    x = synth.normal_bf16((T, D), 30.0, 0, "head_full_x")
    out = torch.empty((T, V), dtype=torch.float32, device="cuda")
    B.beam_lm_head_softcap(T, D, V, dev(x), w, 30.0, out)
    B.beam_check()
    g = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, V - 1], g.choice(V, 4096, replace=False)]))
    wr = host_bits(w[torch.from_numpy(rows).cuda()])
    _check(out.cpu().numpy()[:, rows], bf16_bits_to_f64(x), wr, 30.0)
