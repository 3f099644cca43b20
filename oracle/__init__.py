"""CPU oracle for the Beam sparse decoder layer.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call anything under oracle/. The product path
(moe_decoder_layer_amd and its HIP library) never does, and shares no code,
header, table or constant generator with it.

Plain float64 NumPy, stage by stage, each function citing the page section it
follows (see oracle/layer.py). The seeded inputs come from the separate synth/
module, which holds none of the layer's arithmetic.

Pins: tests/test_oracle_*.py check these functions against closed forms,
library routines used as special cases, exhaustive codec enumeration and
float64 brute force on tiny shapes. The composition of the whole layer has no
worked example on the pages: parity unpinned beyond its stages, which are
each pinned, and the invariants (chunking, MoE <-> dense identity) tested.
"""
from . import accounting, layer, mx, numerics  # noqa: F401
from .layer import (KVCache, attention, boundary, dense_ffn, kv_write,  # noqa: F401
                    layer_forward, moe, o_proj, output_gate, qk_norm_position,
                    qkvg_projection, rms_norm, rope, router, scaled_residual,
                    split_qkvg, ssmax_factor, swiglu_ffn)
