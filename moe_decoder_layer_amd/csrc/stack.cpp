// The decoder stack at decode time: the layer schedule of the Beam model and
// one token's step through a run of layers ("Reflection Beam 1.0 on vLLM":
// model architecture, 52 layers of hidden 5120; Attention section, 43
// sliding-window layers and 9 full-context NoPE layers; MoE and residual
// stream section, dense layers 0-2 and the sandwich residual numbered over
// the 104 sublayer boundaries). Host code only: each layer is the composition
// of the single-layer calls, launched in order on one stream, so a caller can
// capture a whole step in one HIP graph.
#include <algorithm>

#include "beamlayer.h"
#include "internal.h"

namespace {

constexpr int kDenseLayers = 3;  // layers 0..2 run a dense SwiGLU FFN

size_t al256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace of a step: one region shared by the layer calls (each leaves its
// counter block at zero and uses the rest only while it runs, and the calls
// run in stream order), then the step's activations.
struct StackWs {
  size_t call, z, y, x2, y2, idx, w, total;
};

bool stack_ws(const beam_dims* d, int Fd, int max_ctx, StackWs* s) {
  beam_dims dd = *d;
  dd.F = Fd;
  const size_t parts[] = {beam_workspace_size(d, BEAM_OP_ATTN_DECODE_FUSED, 1, max_ctx),
                          beam_workspace_size(d, BEAM_OP_OUT_GATE, 1, 0),
                          beam_workspace_size(d, BEAM_OP_ROUTER, 1, 0),
                          beam_workspace_size(d, BEAM_OP_MOE, 1, 0),
                          Fd > 0 ? beam_workspace_size(&dd, BEAM_OP_DENSE, 1, 0) : 0};
  size_t call = 0;
  for (size_t p : parts) {
    if (p == (size_t)-1) return false;
    call = std::max(call, p);
  }
  s->call = al256(call);
  s->z = s->call;
  s->y = s->z + al256((size_t)d->Hq * d->d * 2);
  s->x2 = s->y + al256((size_t)d->D * 2);
  s->y2 = s->x2 + al256((size_t)d->D * 2);
  s->idx = s->y2 + al256((size_t)d->D * 2);
  s->w = s->idx + al256((size_t)std::max(d->topk, 1) * 4);
  s->total = s->w + al256((size_t)std::max(d->topk, 1) * 4);
  return true;
}

}  // namespace

extern "C" {

int beam_layer_kind(int layer, int n_layers, int* attn_mode, int* dense) {
  if (!attn_mode || !dense) return beam::abi_fail(BEAM_E_NULL, "%s: NULL output", __func__);
  if (n_layers <= 0 || layer < 0 || layer >= n_layers)
    return beam::abi_fail(BEAM_E_SHAPE, "%s: layer %d outside [0, %d)", __func__, layer,
                          n_layers);
  // full context without positions on every sixth layer (1-based) and the last
  const bool nope = (layer + 1) % 6 == 0 || layer == n_layers - 1;
  *attn_mode = nope ? BEAM_NOPE_SSMAX : BEAM_SWA_ROPE;
  *dense = layer < kDenseLayers ? 1 : 0;
  return BEAM_OK;
}

size_t beam_decode_stack_workspace(const beam_dims* dims, int Fd, int max_ctx) {
  StackWs s;
  if (!dims || max_ctx <= 0 || Fd < 0 || !stack_ws(dims, Fd, max_ctx, &s)) return (size_t)-1;
  return s.total;
}

int beam_decode_stack(const beam_dims* dims, int Fd, int layer0, int n_layers,
                      const beam_stack_layer* layers, const uint16_t* w_final, uint16_t* h,
                      uint16_t* x_out, const int32_t* pos, const int32_t* seq,
                      const float* rope_cs, int max_pos, void* ws, size_t ws_bytes,
                      void* stream) {
  using beam::abi_fail;
  if (!dims || !layers || !w_final || !h || !x_out || !pos || !seq || !ws)
    return abi_fail(BEAM_E_NULL, "%s: NULL argument", __func__);
  if (n_layers <= 0 || layer0 < 0)
    return abi_fail(BEAM_E_SHAPE, "%s: n_layers %d, layer0 %d", __func__, n_layers, layer0);
  if (max_pos < 0) return abi_fail(BEAM_E_SHAPE, "%s: max_pos < 0", __func__);
  StackWs s;
  if (Fd < 0 || !stack_ws(dims, Fd, max_pos + 1, &s))
    return abi_fail(BEAM_E_SHAPE, "%s: invalid dims", __func__);
  if (ws_bytes < s.total)
    return abi_fail(BEAM_E_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes,
                    s.total);
  for (int l = 0; l < n_layers; ++l) {
    const beam_stack_layer& L = layers[l];
    if (L.attn_mode != BEAM_SWA_ROPE && L.attn_mode != BEAM_NOPE_SSMAX)
      return abi_fail(BEAM_E_SHAPE, "%s: layer %d: invalid attention mode", __func__, l);
    if (L.dense && Fd <= 0)
      return abi_fail(BEAM_E_SHAPE, "%s: layer %d is dense but Fd = %d", __func__, l, Fd);
    if (!L.dense && (!L.w_r || !L.b_corr))
      return abi_fail(BEAM_E_NULL, "%s: layer %d: MoE layer without router", __func__, l);
  }
  char* base = (char*)ws;
  void* wcall = base;
  uint16_t* z = (uint16_t*)(base + s.z);
  uint16_t* y = (uint16_t*)(base + s.y);
  uint16_t* x2 = (uint16_t*)(base + s.x2);
  uint16_t* y2 = (uint16_t*)(base + s.y2);
  int32_t* idx = (int32_t*)(base + s.idx);
  float* w = (float*)(base + s.w);
  int rc = beam_boundary_norm_residual(dims, 1, nullptr, nullptr, h, layers[0].w_attn_pre, x_out,
                                       0, stream);
  for (int l = 0; l < n_layers && rc == BEAM_OK; ++l) {
    const beam_stack_layer& L = layers[l];
    const int n = 2 * (layer0 + l) + 1;  // the layer's two residual adds: n and n + 1
    const uint16_t* w_next = (l + 1 < n_layers) ? layers[l + 1].w_attn_pre : w_final;
    // attention half: projection, q/k epilogue with the cache write,
    // attention and the output gate in one call, then o_proj
    rc = beam_attn_decode_fused(dims, 1, x_out, L.w_qkvg, L.w_qnorm, L.w_knorm, pos, seq,
                                L.attn_mode, L.attn_mode == BEAM_SWA_ROPE ? rope_cs : nullptr,
                                &L.kv, nullptr, L.b_gate, nullptr, z, max_pos, wcall,
                                s.call, stream);
    if (rc) break;
    rc = beam_out_gate(dims, 1, z, nullptr, nullptr, L.w_o, y, wcall, s.call, stream);
    if (rc) break;
    // FFN half: the attention-side boundary (with the router on MoE layers),
    // the FFN, and the FFN-side boundary that forms the next layer's input
    if (L.dense) {
      rc = beam_boundary_norm_residual(dims, 1, y, L.w_attn_post, h, L.w_ffn_pre, x2, n, stream);
      if (rc) break;
      rc = beam_dense_swiglu(1, dims->D, Fd, x2, L.w13, L.w2, y2, wcall, s.call, stream);
    } else {
      rc = beam_boundary_router_fp32_grouped_topk(dims, 1, y, L.w_attn_post, h, L.w_ffn_pre, x2,
                                                  n, L.w_r, L.b_corr, idx, w, nullptr, wcall,
                                                  s.call, stream);
      if (rc) break;
      rc = beam_moe_swiglu_combine(dims, 1, x2, idx, w, L.w13, L.w2, nullptr, nullptr, y2, wcall,
                                   s.call, stream);
    }
    if (rc) break;
    rc = beam_boundary_norm_residual(dims, 1, y2, L.w_ffn_post, h, w_next, x_out, n + 1, stream);
  }
  return rc;
}

}  // extern "C"
