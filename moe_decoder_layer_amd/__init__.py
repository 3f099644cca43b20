"""Python binding of libbeamlayer (the C ABI in include/beamlayer.h).

Argument marshalling only: every function forwards to the C call of the same
name, turning torch tensors into device pointers and the layer shape into a
beam_dims struct; all computation happens in the library's HIP kernels. A
non-zero status raises BeamError with the library's message. The default
stream is torch's current stream, so calls compose with torch work and with
graph capture.

The shared library must have been built (python -m moe_decoder_layer_amd.build);
importing works without it, the first call fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_double, c_float, c_int, c_size_t, c_void_p

__all__ = [
    "BeamError", "beam_dims", "beam_kv", "lib", "dims_from", "kv_struct",
    "beam_boundary_norm_residual", "beam_qk_norm_rope_ssmax_kvwrite", "beam_attn_swa",
    "beam_attn_nope_ssmax", "beam_out_gate", "beam_router_fp32_grouped_topk",
    "beam_boundary_router_fp32_grouped_topk",
    "beam_moe_swiglu_combine", "beam_moe_experts_up", "beam_moe_experts_down",
    "beam_dense_swiglu", "beam_workspace_size", "beam_rope_table", "beam_hbm_read",
    "beam_mxfp8_quantize", "beam_moe_swiglu_combine_mxfp8",
    "beam_mxfp4_quantize", "beam_moe_swiglu_combine_mxfp4", "beam_lm_head_softcap",
    "beam_check", "beam_last_error", "beam_version",
    "BEAM_SWA_ROPE", "BEAM_NOPE_SSMAX", "BEAM_KV_BF16", "BEAM_KV_FP8_E4M3",
    "BEAM_OP_QKV", "BEAM_OP_ATTN_SWA", "BEAM_OP_ATTN_NOPE", "BEAM_OP_OUT_GATE",
    "BEAM_OP_ROUTER", "BEAM_OP_MOE", "BEAM_OP_DENSE", "BEAM_OP_ATTN_DECODE_FUSED",
    "BEAM_OP_MOE_MX_SCALED", "beam_moe_swiglu_combine_mx_scaled", "LIB_PATH",
    "HEADER_PATH",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbeamlayer.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "beamlayer.h")

BEAM_SWA_ROPE, BEAM_NOPE_SSMAX = 0, 1
BEAM_KV_BF16, BEAM_KV_FP8_E4M3 = 0, 1
(BEAM_OP_QKV, BEAM_OP_ATTN_SWA, BEAM_OP_ATTN_NOPE, BEAM_OP_OUT_GATE, BEAM_OP_ROUTER,
 BEAM_OP_MOE, BEAM_OP_DENSE, BEAM_OP_ATTN_DECODE_FUSED, BEAM_OP_MOE_MX_SCALED) = range(1, 10)


class BeamError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class beam_dims(ctypes.Structure):
    _fields_ = [(n, c_int) for n in ("D", "Hq", "Hkv", "d", "G", "E", "n_group",
                                      "topk_group", "topk", "F", "window")] + \
               [("eps", c_float), ("route_scale", c_float)]


class beam_kv(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("dtype", c_int), ("k_scale", c_float),
                ("v_scale", c_float), ("S", c_int), ("Lmax", c_int), ("npos", c_int)]


class beam_stack_layer(ctypes.Structure):
    _fields_ = [("attn_mode", c_int), ("dense", c_int)] + \
               [(n, c_void_p) for n in ("w_attn_pre", "w_attn_post", "w_ffn_pre", "w_ffn_post",
                                        "w_qnorm", "w_knorm", "w_qkvg", "b_gate", "w_o", "w_r",
                                        "b_corr", "w13", "w2")] + [("kv", beam_kv)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m moe_decoder_layer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = c_void_p
        sig = {
            "beam_boundary_norm_residual": [POINTER(beam_dims), c_int, P, P, P, P, P, c_int, P],
            "beam_qk_norm_rope_ssmax_kvwrite": [POINTER(beam_dims), c_int, P, P, P, P, P, P,
                                                c_int, P, P, P, POINTER(beam_kv), P, c_size_t, P],
            "beam_attn_swa": [POINTER(beam_dims), c_int, P, P, P, POINTER(beam_kv), P, P, c_int,
                              P, c_size_t, P],
            "beam_attn_nope_ssmax": [POINTER(beam_dims), c_int, P, P, P, POINTER(beam_kv), P, P,
                                     c_int, P, c_size_t, P],
            "beam_attn_nope_ssmax_static": [POINTER(beam_dims), c_int, P, P, P, POINTER(beam_kv),
                                            P, P, c_int, P],
            "beam_attn_decode_fused": [POINTER(beam_dims), c_int, P, P, P, P, P, P, c_int, P,
                                       POINTER(beam_kv), P, P, P, P, c_int, P, c_size_t, P],
            "beam_out_gate": [POINTER(beam_dims), c_int, P, P, P, P, P, P, c_size_t, P],
            "beam_router_fp32_grouped_topk": [POINTER(beam_dims), c_int, P, P, P, P, P, P, P,
                                              c_size_t, P],
            "beam_boundary_router_fp32_grouped_topk": [POINTER(beam_dims), c_int, P, P, P, P, P,
                                                       c_int, P, P, P, P, P, P, c_size_t, P],
            "beam_moe_swiglu_combine": [POINTER(beam_dims), c_int, P, P, P, P, P, P, P, P, P,
                                        c_size_t, P],
            "beam_moe_experts_up": [POINTER(beam_dims), c_int, P, P, P, P, P, P],
            "beam_moe_experts_down": [POINTER(beam_dims), c_int, P, P, P, P, P, P, P],
            "beam_dense_swiglu": [c_int, c_int, c_int, P, P, P, P, P, c_size_t, P],
            "beam_rope_table": [P, c_int, c_int, c_double],
            "beam_hbm_read": [P, c_size_t, P, P],
            "beam_mxfp8_quantize": [P, c_size_t, c_int, P, P, P],
            "beam_moe_swiglu_combine_mxfp8": [POINTER(beam_dims), c_int, P, P, P, P, P, P, P, P,
                                              P, c_size_t, P],
            "beam_mxfp4_quantize": [P, c_size_t, c_int, P, P, P],
            "beam_lm_head_softcap": [c_int, c_int, c_int, P, P, c_float, P, P],
            "beam_moe_swiglu_combine_mxfp4": [POINTER(beam_dims), c_int, P, P, P, P, P, P, P, P,
                                              P, c_size_t, P],
            "beam_moe_swiglu_combine_mx_scaled": [POINTER(beam_dims), c_int, P, P, P, c_int,
                                                  P, P, P, P, P, P, c_size_t, P],
            "beam_layer_kind": [c_int, c_int, POINTER(c_int), POINTER(c_int)],
            "beam_decode_stack": [POINTER(beam_dims), c_int, c_int, c_int,
                                  POINTER(beam_stack_layer), P, P, P, P, P, P, c_int, P,
                                  c_size_t, P],
            "beam_check": [P],
            "beam_version": [],
            "beam_last_error": [],
        }
        for name, args in sig.items():
            f = getattr(L, name, None)
            if f is None:  # absent from this build: calling it raises AttributeError
                continue
            f.argtypes = args
            f.restype = c_int
        L.beam_last_error.restype = ctypes.c_char_p
        L.beam_workspace_size.argtypes = [POINTER(beam_dims), c_int, c_int, c_int]
        L.beam_workspace_size.restype = c_size_t
        if hasattr(L, "beam_decode_stack_workspace"):
            L.beam_decode_stack_workspace.argtypes = [POINTER(beam_dims), c_int, c_int]
            L.beam_decode_stack_workspace.restype = c_size_t
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/beamlayer.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(beam_[a-z0-9_]+)\s*\(", text)))


# ---------------------------------------------------------------- marshalling
def dims_from(obj) -> beam_dims:
    """beam_dims from any object (or dict) with the fields D, Hq, Hkv, d, G, E,
    n_group, topk_group, topk, F, window, eps, route_scale."""
    get = obj.__getitem__ if isinstance(obj, dict) else lambda k: getattr(obj, k)
    return beam_dims(*(int(get(n)) for n in ("D", "Hq", "Hkv", "d", "G", "E", "n_group",
                                             "topk_group", "topk", "F", "window")),
                     float(get("eps")), float(get("route_scale")))


def kv_struct(k, v, dtype: int, k_scale: float, v_scale: float, S: int, Lmax: int,
              npos: int = 0) -> beam_kv:
    """npos > Lmax: a ring of Lmax slots per sequence (slot = position mod Lmax)."""
    return beam_kv(_p(k), _p(v), dtype, k_scale, v_scale, S, Lmax, npos)


def _p(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _d(dims):
    return dims if isinstance(dims, beam_dims) else dims_from(dims)


def _ws(ws):
    if ws is None:
        return None, 0
    return _p(ws), ws.numel() * ws.element_size()


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise BeamError(rc, lib().beam_last_error().decode())


# ---------------------------------------------------------------- entry points
def beam_boundary_norm_residual(dims, T, y, w_post, h, w_pre, x_out, n, stream=None):
    d = _d(dims)
    _call("beam_boundary_norm_residual", ctypes.byref(d), T, _p(y), _p(w_post), _p(h),
          _p(w_pre), _p(x_out), n, _s(stream))


def beam_qk_norm_rope_ssmax_kvwrite(dims, T, x, w_qkvg, w_qnorm, w_knorm, pos, seq, mode,
                                    rope_cs, q_out, g_out, kv: beam_kv, ws, stream=None):
    d = _d(dims)
    wp, wb = _ws(ws)
    _call("beam_qk_norm_rope_ssmax_kvwrite", ctypes.byref(d), T, _p(x), _p(w_qkvg),
          _p(w_qnorm), _p(w_knorm), _p(pos), _p(seq), mode, _p(rope_cs), _p(q_out), _p(g_out),
          ctypes.byref(kv), wp, wb, _s(stream))


def beam_attn_swa(dims, T, q, pos, seq, kv: beam_kv, sink, o, max_pos, ws, stream=None):
    d = _d(dims)
    wp, wb = _ws(ws)
    _call("beam_attn_swa", ctypes.byref(d), T, _p(q), _p(pos), _p(seq), ctypes.byref(kv),
          _p(sink), _p(o), max_pos, wp, wb, _s(stream))


def beam_attn_nope_ssmax(dims, T, q, pos, seq, kv: beam_kv, sink, o, max_pos, ws, stream=None):
    d = _d(dims)
    wp, wb = _ws(ws)
    _call("beam_attn_nope_ssmax", ctypes.byref(d), T, _p(q), _p(pos), _p(seq),
          ctypes.byref(kv), _p(sink), _p(o), max_pos, wp, wb, _s(stream))


def beam_attn_decode_fused(dims, T, x, w_qkvg, w_qnorm, w_knorm, pos, seq, mode, rope_cs,
                           kv: beam_kv, sink, b_gate, q_out, z_out, max_pos, ws, stream=None):
    d = _d(dims)
    wp, wb = _ws(ws)
    _call("beam_attn_decode_fused", ctypes.byref(d), T, _p(x), _p(w_qkvg), _p(w_qnorm),
          _p(w_knorm), _p(pos), _p(seq), mode, _p(rope_cs), ctypes.byref(kv), _p(sink),
          _p(b_gate), _p(q_out), _p(z_out), max_pos, wp, wb, _s(stream))


def beam_attn_nope_ssmax_static(dims, T, q, pos, seq, kv: beam_kv, sink, o, max_pos,
                                stream=None):
    d = _d(dims)
    _call("beam_attn_nope_ssmax_static", ctypes.byref(d), T, _p(q), _p(pos), _p(seq),
          ctypes.byref(kv), _p(sink), _p(o), max_pos, _s(stream))


def beam_out_gate(dims, T, o, g, b_gate, w_o, y, ws=None, stream=None):
    d = _d(dims)
    wp, wb = _ws(ws)
    _call("beam_out_gate", ctypes.byref(d), T, _p(o), _p(g), _p(b_gate), _p(w_o), _p(y), wp, wb,
          _s(stream))


def beam_router_fp32_grouped_topk(dims, T, x, w_r, b_corr, idx, w, logits=None, ws=None,
                                  stream=None):
    d = _d(dims)
    wp, wb = _ws(ws)
    _call("beam_router_fp32_grouped_topk", ctypes.byref(d), T, _p(x), _p(w_r), _p(b_corr),
          _p(idx), _p(w), _p(logits), wp, wb, _s(stream))


def beam_boundary_router_fp32_grouped_topk(dims, T, y, w_post, h, w_pre, x_out, n, w_r, b_corr,
                                           idx, w, logits=None, ws=None, stream=None):
    d = _d(dims)
    wp, wb = _ws(ws)
    _call("beam_boundary_router_fp32_grouped_topk", ctypes.byref(d), T, _p(y), _p(w_post), _p(h),
          _p(w_pre), _p(x_out), n, _p(w_r), _p(b_corr), _p(idx), _p(w), _p(logits), wp, wb,
          _s(stream))


def beam_moe_swiglu_combine(dims, T, x, idx, w, w13, w2, shared_w13, shared_w2, y, ws,
                            stream=None):
    d = _d(dims)
    wp, wb = _ws(ws)
    _call("beam_moe_swiglu_combine", ctypes.byref(d), T, _p(x), _p(idx), _p(w), _p(w13),
          _p(w2), _p(shared_w13), _p(shared_w2), _p(y), wp, wb, _s(stream))


def beam_moe_experts_up(dims, T, x, idx, w13, shared_w13, act, stream=None):
    d = _d(dims)
    _call("beam_moe_experts_up", ctypes.byref(d), T, _p(x), _p(idx), _p(w13), _p(shared_w13),
          _p(act), _s(stream))


def beam_moe_experts_down(dims, T, idx, w, w2, shared_w2, act, y, stream=None):
    d = _d(dims)
    _call("beam_moe_experts_down", ctypes.byref(d), T, _p(idx), _p(w), _p(w2), _p(shared_w2),
          _p(act), _p(y), _s(stream))


def beam_dense_swiglu(T, D, Fd, x, w13, w2, y, ws, stream=None):
    wp, wb = _ws(ws)
    _call("beam_dense_swiglu", T, D, Fd, _p(x), _p(w13), _p(w2), _p(y), wp, wb, _s(stream))


def beam_mxfp8_quantize(w, rows, K, codes, scales, stream=None):
    _call("beam_mxfp8_quantize", _p(w), rows, K, _p(codes), _p(scales), _s(stream))


def beam_moe_swiglu_combine_mxfp8(dims, T, x, idx, w, w13_codes, w13_scales, w2_codes,
                                  w2_scales, y, ws, stream=None):
    d = _d(dims)
    wp, wb = _ws(ws)
    _call("beam_moe_swiglu_combine_mxfp8", ctypes.byref(d), T, _p(x), _p(idx), _p(w),
          _p(w13_codes), _p(w13_scales), _p(w2_codes), _p(w2_scales), _p(y), wp, wb, _s(stream))


def beam_mxfp4_quantize(w, rows, K, codes, scales, stream=None):
    _call("beam_mxfp4_quantize", _p(w), rows, K, _p(codes), _p(scales), _s(stream))


def beam_moe_swiglu_combine_mxfp4(dims, T, x, idx, w, w13_codes, w13_scales, w2_codes,
                                  w2_scales, y, ws, stream=None):
    d = _d(dims)
    wp, wb = _ws(ws)
    _call("beam_moe_swiglu_combine_mxfp4", ctypes.byref(d), T, _p(x), _p(idx), _p(w),
          _p(w13_codes), _p(w13_scales), _p(w2_codes), _p(w2_scales), _p(y), wp, wb, _s(stream))


def beam_moe_swiglu_combine_mx_scaled(dims, T, x, idx, w, wbits, w13_codes, w13_scales,
                                      w2_codes, w2_scales, y, ws, stream=None):
    d = _d(dims)
    wp, wb = _ws(ws)
    _call("beam_moe_swiglu_combine_mx_scaled", ctypes.byref(d), T, _p(x), _p(idx), _p(w), wbits,
          _p(w13_codes), _p(w13_scales), _p(w2_codes), _p(w2_scales), _p(y), wp, wb, _s(stream))


def stack_layer(attn_mode: int, dense: int, w: dict, kv: beam_kv) -> beam_stack_layer:
    """One beam_stack_layer from a dict of device tensors (keys as the struct's
    pointer fields; w13/w2 the experts, or the dense FFN when dense=1)."""
    ptrs = [_p(w.get(n)) for n in ("w_attn_pre", "w_attn_post", "w_ffn_pre", "w_ffn_post",
                                   "w_qnorm", "w_knorm", "w_qkvg", "b_gate", "w_o", "w_r",
                                   "b_corr", "w13", "w2")]
    return beam_stack_layer(attn_mode, dense, *ptrs, kv)


def beam_layer_kind(layer, n_layers):
    """(attention mode, dense) of a 0-based layer of an n_layers stack."""
    m, d = ctypes.c_int(), ctypes.c_int()
    _call("beam_layer_kind", layer, n_layers, ctypes.byref(m), ctypes.byref(d))
    return m.value, d.value


def beam_decode_stack_workspace(dims, Fd, max_ctx):
    return lib().beam_decode_stack_workspace(ctypes.byref(_d(dims)), Fd, max_ctx)


def beam_decode_stack(dims, Fd, layer0, layers, w_final, h, x_out, pos, seq, rope_cs, max_pos,
                      ws, stream=None):
    """layers: a sequence of beam_stack_layer (see stack_layer)."""
    d = _d(dims)
    arr = (beam_stack_layer * len(layers))(*layers)
    wp, wb = _ws(ws)
    _call("beam_decode_stack", ctypes.byref(d), Fd, layer0, len(layers), arr, _p(w_final), _p(h),
          _p(x_out), _p(pos), _p(seq), _p(rope_cs), max_pos, wp, wb, _s(stream))


def beam_lm_head_softcap(T, D, V, x, w, cap, logits, stream=None):
    _call("beam_lm_head_softcap", T, D, V, _p(x), _p(w), cap, _p(logits), _s(stream))


def beam_hbm_read(buf, sink, stream=None):
    """Read a device buffer once (HBM streaming-read measurement)."""
    _call("beam_hbm_read", _p(buf), buf.numel() * buf.element_size(), _p(sink), _s(stream))


def beam_workspace_size(dims, op, T, max_ctx=0) -> int:
    d = _d(dims)
    n = lib().beam_workspace_size(ctypes.byref(d), op, T, max_ctx)
    if n == ctypes.c_size_t(-1).value:
        raise BeamError(-2, "beam_workspace_size: invalid arguments")
    return n


def beam_rope_table(out, Lmax, d, theta):
    """Fill a host float32 buffer (numpy array or torch CPU tensor) [Lmax][d]."""
    ptr = out.ctypes.data if hasattr(out, "ctypes") else out.data_ptr()
    _call("beam_rope_table", ptr, Lmax, d, theta)


def beam_check(stream=None):
    _call("beam_check", _s(stream))


def beam_last_error() -> str:
    return lib().beam_last_error().decode()


def beam_version() -> int:
    return lib().beam_version()
