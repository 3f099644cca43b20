"""The C-ABI library: loads, exports what the header declares, and rejects bad
arguments on the host before any HIP call (no GPU needed)."""
import ctypes

import numpy as np
import pytest
import torch

import moe_decoder_layer_amd as B
import synth

NO_GPU = not torch.cuda.is_available()
# Fake device addresses are only ever passed to calls that must fail
# validation (or find no device); never run these where a GPU is present.
cpu_only = pytest.mark.skipif(not NO_GPU, reason="fake-pointer checks run on GPU-less hosts only")

A = 0x10000          # a 16-byte aligned fake address
MIS = 0x10002        # misaligned


def test_library_exports_every_declared_symbol():
    names = B.header_functions()
    assert len(names) == 28
    L = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert B.beam_version() == 100


def _dims(i=0, **kw):
    d = synth.with_dims(synth.config(i), **kw).dims
    return B.dims_from(d)


def _rc(name, *args):
    return getattr(B.lib(), name)(*args)


@cpu_only
def test_boundary_validation_and_nodev():
    d = _dims()
    by = ctypes.byref(d)
    assert _rc("beam_boundary_norm_residual", by, 1, A, A, None, A, A, 5, None) == -1
    assert _rc("beam_boundary_norm_residual", None, 1, A, A, A, A, A, 5, None) == -1
    assert _rc("beam_boundary_norm_residual", by, 0, A, A, A, A, A, 5, None) == -2
    assert _rc("beam_boundary_norm_residual", by, 1, A, A, A, A, A, -1, None) == -2
    assert _rc("beam_boundary_norm_residual", by, 1, MIS, A, A, A, A, 5, None) == -4
    bad = _dims(D=250)
    assert _rc("beam_boundary_norm_residual", ctypes.byref(bad), 1, A, A, A, A, A, 5, None) == -3
    assert _rc("beam_boundary_norm_residual", by, 1, A, A, A, A, A, 5, None) == -7
    assert "device" in B.beam_last_error()


@cpu_only
def test_qkv_validation():
    d = _dims()
    by = ctypes.byref(d)
    kv = B.kv_struct(A, A, B.BEAM_KV_BF16, 1.0, 1.0, 1, 128)
    ws = B.beam_workspace_size(d, B.BEAM_OP_QKV, 1)
    args = lambda **o: [by, o.get("T", 1), A, A, A, A, A, A, o.get("mode", 0),  # noqa: E731
                        o.get("rope", A), A, A, ctypes.byref(o.get("kv", kv)), A,
                        o.get("ws", ws), None]
    assert _rc("beam_qk_norm_rope_ssmax_kvwrite", *args(mode=7)) == -2
    assert _rc("beam_qk_norm_rope_ssmax_kvwrite", *args(rope=None)) == -1
    assert _rc("beam_qk_norm_rope_ssmax_kvwrite", *args(ws=ws - 1)) == -5
    kv8 = B.kv_struct(A, A, B.BEAM_KV_FP8_E4M3, 0.0, 1.0, 1, 128)
    assert _rc("beam_qk_norm_rope_ssmax_kvwrite", *args(kv=kv8)) == -2
    kvL = B.kv_struct(A, A, B.BEAM_KV_BF16, 1.0, 1.0, 1, 100)
    assert _rc("beam_qk_norm_rope_ssmax_kvwrite", *args(kv=kvL)) == -2
    d2 = _dims(Hkv=3)
    a2 = args()
    a2[0] = ctypes.byref(d2)
    assert _rc("beam_qk_norm_rope_ssmax_kvwrite", *a2) == -2
    d3 = _dims(d=48)
    a3 = args()
    a3[0] = ctypes.byref(d3)
    assert _rc("beam_qk_norm_rope_ssmax_kvwrite", *a3) == -3
    assert _rc("beam_qk_norm_rope_ssmax_kvwrite", *args()) == -7


@cpu_only
def test_attention_router_moe_validation():
    d = _dims()
    by = ctypes.byref(d)
    kv = B.kv_struct(A, A, B.BEAM_KV_BF16, 1.0, 1.0, 1, 8192)
    ws = B.beam_workspace_size(d, B.BEAM_OP_ATTN_NOPE, 1, 8000)
    assert _rc("beam_attn_nope_ssmax", by, 1, A, A, A, ctypes.byref(kv), None, A, 8192, A, ws,
               None) == -2                                     # max_pos >= Lmax
    # a long context is split over workgroups and needs the partials workspace
    assert _rc("beam_attn_nope_ssmax", by, 1, A, A, A, ctypes.byref(kv), None, A, 7999, A, 16,
               None) == -5
    assert _rc("beam_attn_nope_ssmax", by, 1, A, A, A, ctypes.byref(kv), None, A, 7999, None, 0,
               None) == -1
    assert _rc("beam_attn_nope_ssmax", by, 1, A, A, A, ctypes.byref(kv), None, A, 7999, A, ws,
               None) == -7
    # a short one is taken in one pass and needs only the counter block
    assert _rc("beam_attn_nope_ssmax", by, 1, A, A, A, ctypes.byref(kv), None, A, 64, None, 0,
               None) == -1
    assert _rc("beam_attn_nope_ssmax", by, 1, A, A, A, ctypes.byref(kv), None, A, 64, A, 1024,
               None) == -7
    dw = _dims(window=0)
    assert _rc("beam_attn_swa", ctypes.byref(dw), 1, A, A, A, ctypes.byref(kv), None, A, 64, A,
               ws, None) == -2
    # ring caches (slot = position mod Lmax): npos above Lmax, sliding window only,
    # window inside the ring, max_pos below npos
    ring = B.kv_struct(A, A, B.BEAM_KV_BF16, 1.0, 1.0, 1, 512, 1 << 20)
    wsr = B.beam_workspace_size(d, B.BEAM_OP_ATTN_SWA, 1, 1 << 20)
    assert _rc("beam_attn_swa", by, 1, A, A, A, ctypes.byref(ring), None, A, 900000, A, wsr,
               None) == -7                                     # accepted (no device here)
    assert _rc("beam_attn_swa", by, 1, A, A, A, ctypes.byref(ring), None, A, 1 << 20, A, wsr,
               None) == -2                                     # max_pos >= npos
    assert _rc("beam_attn_nope_ssmax", by, 1, A, A, A, ctypes.byref(ring), None, A, 900, A,
               wsr, None) == -3                                # full context on a ring
    assert _rc("beam_attn_nope_ssmax_static", by, 1, A, A, A, ctypes.byref(ring), None, A, 900,
               None) == -3
    small = B.kv_struct(A, A, B.BEAM_KV_BF16, 1.0, 1.0, 1, 448, 1 << 20)
    d512 = _dims(window=512)
    assert _rc("beam_attn_swa", ctypes.byref(d512), 1, A, A, A, ctypes.byref(small), None, A,
               900, A, wsr, None) == -2                        # window 512 > 448 slots
    part = B.kv_struct(A, A, B.BEAM_KV_BF16, 1.0, 1.0, 1, 512, 300)
    assert _rc("beam_attn_swa", by, 1, A, A, A, ctypes.byref(part), None, A, 200, A, wsr,
               None) == -2                                     # 0 < npos < Lmax
    # router: topk larger than the kept groups can hold
    dr = _dims(topk=9)
    assert _rc("beam_router_fp32_grouped_topk", ctypes.byref(dr), 1, A, A, None, A, A, A, None,
               0, None) == -2
    dr = _dims(E=15)
    assert _rc("beam_router_fp32_grouped_topk", ctypes.byref(dr), 1, A, A, None, A, A, A, None,
               0, None) == -2
    assert _rc("beam_router_fp32_grouped_topk", by, 1, A, A, None, A, A, None, A, 16,
               None) == -5
    # the counter block is needed even when the logits are an output
    assert _rc("beam_router_fp32_grouped_topk", by, 1, A, A, None, A, A, A, None, 0, None) == -1
    assert _rc("beam_router_fp32_grouped_topk", by, 1, A, A, None, A, A, A, A, 1023,
               None) == -5
    assert _rc("beam_router_fp32_grouped_topk", by, 1, A, A, None, A, A, A, A, 1024,
               None) == -7
    wsm = B.beam_workspace_size(d, B.BEAM_OP_MOE, 1)
    assert _rc("beam_moe_swiglu_combine", by, 1, A, A, A, A, A, A, None, A, A, wsm, None) == -1
    assert _rc("beam_moe_swiglu_combine", by, 1, A, A, A, A, A, None, None, A, A, wsm - 256,
               None) == -5
    assert _rc("beam_moe_swiglu_combine", by, 1, A, A, A, A, A, None, None, A, A, wsm,
               None) == -7
    assert _rc("beam_dense_swiglu", 1, 256, 100, A, A, A, A, A, 1 << 20, None) == -2
    assert _rc("beam_dense_swiglu", 1, 256, 512, A, A, A, A, A, 1 << 20, None) == -7
    assert _rc("beam_out_gate", by, 1, A, A, None, A, A, None, 0, None) == -1  # gate, no bias
    assert _rc("beam_out_gate", by, 1, A, None, None, A, A, None, 0, None) == -7  # o_proj alone
    assert _rc("beam_out_gate", by, 1, A, A, A, A, A, None, 0, None) == -7


@cpu_only
def test_hbm_read_validation_and_nodev():
    assert _rc("beam_hbm_read", None, 1024, A, None) == -1
    assert _rc("beam_hbm_read", A, 1024, None, None) == -1
    assert _rc("beam_hbm_read", MIS, 1024, A, None) == -4
    assert _rc("beam_hbm_read", A, 1000, A, None) == -2
    assert _rc("beam_hbm_read", A, 1024, A, None) == -7


def test_workspace_sizes():
    d = _dims(1)
    ctl = 1024  # every workspace starts with the zeroed counter block
    assert B.beam_workspace_size(d, B.BEAM_OP_QKV, 1) >= ctl + (48 + 16) * 128 * 2
    for op in (B.BEAM_OP_OUT_GATE, B.BEAM_OP_ROUTER, B.BEAM_OP_MOE, B.BEAM_OP_DENSE):
        assert B.beam_workspace_size(d, op, 1) >= ctl
    a = B.beam_workspace_size(d, B.BEAM_OP_ATTN_NOPE, 1, 100001)
    s = B.beam_workspace_size(d, B.BEAM_OP_ATTN_SWA, 1, 100001)
    # a 512-key window is split over 3 workgroups per kv head (48 heads x 3 partial
    # records of d + 4 floats); the full context over many more
    assert s == ctl + 48 * 3 * (128 + 4) * 4 and a > s
    # monotone in the context bound
    sizes = [B.beam_workspace_size(d, B.BEAM_OP_ATTN_NOPE, 1, c) for c in range(1000, 200000, 997)]
    assert all(x <= y for x, y in zip(sizes, sizes[1:]))
    with pytest.raises(B.BeamError):
        B.beam_workspace_size(d, 99, 1)


def test_rope_table_host_helper():
    L, dd, theta = 300, 32, 1e4
    out = np.zeros((L, dd), np.float32)
    B.beam_rope_table(out, L, dd, theta)
    p = np.arange(L)[:, None]
    i = np.arange(dd // 2)[None, :]
    ang = p * theta ** (-2.0 * i / dd)
    np.testing.assert_array_equal(out[:, :dd // 2], np.cos(ang).astype(np.float32))
    np.testing.assert_array_equal(out[:, dd // 2:], np.sin(ang).astype(np.float32))
    with pytest.raises(B.BeamError):
        B.beam_rope_table(out, L, 31, theta)

@cpu_only
@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_validation_and_nodev(fmt):
    q, moe = f"beam_{fmt}_quantize", f"beam_moe_swiglu_combine_{fmt}"
    assert _rc(q, None, 4, 64, A, A, None) == -1
    assert _rc(q, A, 4, 48, A, A, None) == -2
    assert _rc(q, MIS, 4, 64, A, A, None) == -4
    assert _rc(q, A, 0, 64, A, A, None) == 0      # nothing to do
    assert _rc(q, A, 4, 64, A, A, None) == -7
    d = _dims()
    by = ctypes.byref(d)
    need = 1024 + 4 * 64 * 2   # counter block + act [1 * topk][F] bf16
    args = lambda T=1, ws=need, dims=by: [dims, T, A, A, A, A, A, A, A, A, A, ws, None]  # noqa
    assert _rc(moe, *args(dims=None)) == -1
    assert _rc(moe, *args(T=0)) == -2
    assert _rc(moe, *args(T=5)) == -3
    d2 = _dims(D=272)
    assert _rc(moe, *args(dims=ctypes.byref(d2))) == -3
    d3 = _dims(F=80)
    assert _rc(moe, *args(dims=ctypes.byref(d3))) == -3
    assert _rc(moe, *args(ws=need - 1)) == -5
    assert _rc(moe, *args()) == -7


@cpu_only
def test_mx_scaled_validation_and_nodev():
    f = "beam_moe_swiglu_combine_mx_scaled"
    d = _dims(D=256, F=128, E=8, topk=2)
    by = ctypes.byref(d)
    T = 300
    need = B.beam_workspace_size(d, B.BEAM_OP_MOE_MX_SCALED, T)
    # staged operands, expert-ordered activations, MXFP8 copies, per-pair fp32 outputs
    P = T * 2
    assert need >= 1024 + P * 4 + T * 256 * (1 + 1 / 32) + P * 128 * (2 + 1 + 1 / 32) + P * 256 * 4

    def args(T=T, wbits=8, scales=A, ws=need, dims=by, x=A):
        return [dims, T, x, A, A, wbits, A, scales, A, A, A, A, ws, None]
    assert _rc(f, *args(dims=None)) == -1
    assert _rc(f, *args(x=None)) == -1
    assert _rc(f, *args(x=MIS)) == -4
    assert _rc(f, *args(scales=A + 2)) == -4
    assert _rc(f, *args(T=0)) == -2
    assert _rc(f, *args(wbits=6)) == -2
    for bad in (dict(D=192), dict(F=192), dict(E=1025)):
        db = _dims(**{**dict(D=256, F=128, E=8, topk=2), **bad})
        assert _rc(f, *args(dims=ctypes.byref(db))) in (-2, -3)
    assert _rc(f, *args(ws=need - 1)) == -5
    assert _rc(f, *args()) == -7


@cpu_only
def test_lm_head_validation_and_nodev():
    f = "beam_lm_head_softcap"
    assert _rc(f, 1, 256, 1000, None, A, ctypes.c_float(30.0), A, None) == -1
    assert _rc(f, 1, 256, 1000, A, A, ctypes.c_float(30.0), MIS, None) == -4
    assert _rc(f, 0, 256, 1000, A, A, ctypes.c_float(30.0), A, None) == -2
    assert _rc(f, 1, 256, 0, A, A, ctypes.c_float(30.0), A, None) == -2
    assert _rc(f, 1, 256, 1000, A, A, ctypes.c_float(-1.0), A, None) == -2
    assert _rc(f, 1, 256, 1000, A, A, ctypes.c_float(float("inf")), A, None) == -2
    assert _rc(f, 1, 260, 1000, A, A, ctypes.c_float(30.0), A, None) == -3
    assert _rc(f, 1, 256, 1000, A, A, ctypes.c_float(30.0), A, None) == -7


@cpu_only
def test_static_attention_validation():
    """The allocation-free attention call rejects, before touching the
    device, a call whose split-K records exceed its static 16 MiB."""
    d = _dims(1)
    by = ctypes.byref(d)
    kv = B.kv_struct(A, A, B.BEAM_KV_BF16, 1.0, 1.0, 128, 131072)
    f = "beam_attn_nope_ssmax_static"
    assert _rc(f, None, 1, A, A, A, ctypes.byref(kv), None, A, 100, None) == -1
    assert _rc(f, by, 0, A, A, A, ctypes.byref(kv), None, A, 100, None) == -2
    assert _rc(f, by, 128, A, A, A, ctypes.byref(kv), None, A, 100000, None) == -5
    assert "static" in B.beam_last_error()
    assert _rc(f, by, 128, A, A, A, ctypes.byref(kv), None, A, 81919, None) == -7  # fits: no device
    assert _rc(f, by, 1, A, A, A, ctypes.byref(kv), None, A, 100000, None) == -7


def test_layer_schedule_matches_oracle():
    """The library's layer schedule (a host helper) against the oracle's, which
    is pinned to the pages' 43 / 9 / 3 / 49 counts."""
    from oracle import accounting as acc
    for n in (52, 7, 12, 13, 1):
        for l in range(n):
            attn, ffn = acc.layer_kind(l, n)
            want = (B.BEAM_NOPE_SSMAX if attn == "nope" else B.BEAM_SWA_ROPE,
                    1 if ffn == "dense" else 0)
            assert B.beam_layer_kind(l, n) == want, (n, l)
    with pytest.raises(B.BeamError):
        B.beam_layer_kind(52, 52)
    with pytest.raises(B.BeamError):
        B.beam_layer_kind(-1, 52)


@cpu_only
def test_decode_stack_validation_and_nodev():
    d = _dims()
    kv = B.kv_struct(A, A, B.BEAM_KV_BF16, 1.0, 1.0, 1, 1024)
    w = {n: A for n in ("w_attn_pre", "w_attn_post", "w_ffn_pre", "w_ffn_post", "w_qnorm",
                        "w_knorm", "w_qkvg", "b_gate", "w_o", "w_r", "b_corr", "w13", "w2")}
    moe = B.stack_layer(B.BEAM_SWA_ROPE, 0, w, kv)
    dense = B.stack_layer(B.BEAM_SWA_ROPE, 1, w, kv)
    need = B.beam_decode_stack_workspace(d, 512, 1024)
    assert 0 < need < (1 << 30)
    arr = lambda *ls: (B.beam_stack_layer * len(ls))(*ls)  # noqa: E731
    call = lambda ls, Fd=512, ws=need: _rc("beam_decode_stack", ctypes.byref(d), Fd, 0, len(ls),  # noqa
                                           arr(*ls), A, A, A, A, A, A, 1000, A, ws, None)
    assert call([dense], Fd=0) == -2                   # dense layer without Fd
    assert call([moe], ws=need - 1) == -5
    bad = B.stack_layer(7, 0, w, kv)
    assert call([bad]) == -2
    w2 = dict(w, w_r=None)
    assert call([B.stack_layer(B.BEAM_SWA_ROPE, 0, w2, kv)]) == -1
    assert call([dense, moe]) == -7                    # valid: no device here
