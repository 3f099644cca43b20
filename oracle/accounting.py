"""Layer schedule and KV-cache footprint of the Beam model, from the counts the
pages state (test infrastructure only; see oracle/__init__.py).

"Reflection Beam 1.0 on vLLM" page:
  * model architecture section: 52 layers, hidden 5120;
  * "Attention" section: 43 sliding-window layers over the last 512 tokens with
    RoPE; the other 9 (every sixth layer, and the last) attend the full
    context without positions; only those 9 keep the whole sequence's KV,
    2 (K and V) x 8 kv heads x 128 values each per token;
  * "MoE and residual stream" section: layers 0-2 are dense SwiGLU MLPs, the
    rest MoE;
  * change 1 of the optimisation list: 104 sublayer boundaries.
"vLLM Day-0 support: Recursive's Flint" page, architecture section: 14
full-context layers, 4 kv heads (head dim 128 as on Beam), 28 KiB/token.
"""
from __future__ import annotations

N_LAYERS = 52
N_DENSE = 3


def nope_layers(n_layers: int = N_LAYERS) -> list[int]:
    """0-based indices of the full-context (NoPE) layers: the layers whose
    1-based number is a multiple of 6, plus the last layer."""
    out = [l for l in range(n_layers) if (l + 1) % 6 == 0]
    if n_layers - 1 not in out:
        out.append(n_layers - 1)
    return out


def layer_kind(layer: int, n_layers: int = N_LAYERS) -> tuple[str, str]:
    """(attention kind 'swa'|'nope', ffn kind 'dense'|'moe') of a 0-based layer."""
    attn = "nope" if layer in nope_layers(n_layers) else "swa"
    return attn, ("dense" if layer < N_DENSE else "moe")


def residual_indices(layer: int) -> tuple[int, int]:
    """Indices n of the two residual adds of a 0-based layer (attention, ffn):
    the adds are numbered 1, 2, ... in order through the stack."""
    return 2 * layer + 1, 2 * layer + 2


def n_boundaries(n_layers: int = N_LAYERS) -> int:
    return 2 * n_layers


def kv_bytes_per_token(n_full_layers: int, n_kv_heads: int, head_dim: int,
                       bytes_per_value: int) -> int:
    """Bytes of cache one token adds across the full-context layers (SWA layers
    keep a bounded window and are not counted)."""
    return n_full_layers * 2 * n_kv_heads * head_dim * bytes_per_value
