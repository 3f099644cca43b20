// C ABI of libbeamlayer: argument validation, workspace accounting and shape
// dispatch to the HIP kernels. See include/beamlayer.h for the contract.
#include "beamlayer.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int device_ready() {
  static std::once_flag once;
  static bool ok = false;
  std::call_once(once, [] {
    int n = 0;
    ok = (hipGetDeviceCount(&n) == hipSuccess && n > 0);
  });
  return ok ? BEAM_OK : fail(BEAM_E_NODEV, "no HIP device available");
}

int launched(int rc, const char* fn) {
  if (rc == 0) return BEAM_OK;
  return fail(BEAM_E_HIP, "%s: kernel launch failed: %s", fn,
              hipGetErrorString(hipGetLastError()));
}

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); }

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

#define REQ(p) \
  if (!(p)) return fail(BEAM_E_NULL, "%s: %s is NULL", __func__, #p)
#define ALN(p) \
  if (misaligned(p)) return fail(BEAM_E_ALIGN, "%s: %s is not 16-byte aligned", __func__, #p)
#define SHAPE(cond, ...) \
  if (!(cond)) return fail(BEAM_E_SHAPE, __VA_ARGS__)
#define UNSUP(cond, ...) \
  if (!(cond)) return fail(BEAM_E_UNSUPPORTED, __VA_ARGS__)

hipStream_t S_(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Checks common to every call that reads a beam_dims.
int check_dims_attn(const beam_dims* d, const char* fn) {
  if (d->D <= 0 || d->Hq <= 0 || d->Hkv <= 0 || d->d <= 0)
    return fail(BEAM_E_SHAPE, "%s: non-positive dimension", fn);
  if (d->Hq % d->Hkv) return fail(BEAM_E_SHAPE, "%s: Hq %% Hkv != 0", fn);
  if (d->Hq / d->Hkv > 16) return fail(BEAM_E_UNSUPPORTED, "%s: GQA group above 16", fn);
  if (d->d != 32 && d->d != 64 && d->d != 128)
    return fail(BEAM_E_UNSUPPORTED, "%s: head dim %d not in {32, 64, 128}", fn, d->d);
  if (d->D % 8 || d->D > 8192) return fail(BEAM_E_UNSUPPORTED, "%s: D must be a multiple of 8 <= 8192", fn);
  if (d->G != 0 && d->G != d->Hq * d->d)
    return fail(BEAM_E_UNSUPPORTED, "%s: gate width must be 0 or Hq*d", fn);
  return BEAM_OK;
}

int check_kv(const beam_kv* kv, const char* fn) {
  if (!kv) return fail(BEAM_E_NULL, "%s: kv is NULL", fn);
  if (!kv->k || !kv->v) return fail(BEAM_E_NULL, "%s: kv->k or kv->v is NULL", fn);
  if (misaligned(kv->k) || misaligned(kv->v))
    return fail(BEAM_E_ALIGN, "%s: cache not 16-byte aligned", fn);
  if (kv->S <= 0 || kv->Lmax <= 0) return fail(BEAM_E_SHAPE, "%s: cache S/Lmax <= 0", fn);
  if (kv->Lmax % 64) return fail(BEAM_E_SHAPE, "%s: Lmax must be a multiple of 64", fn);
  if (kv->dtype != BEAM_KV_BF16 && kv->dtype != BEAM_KV_FP8_E4M3)
    return fail(BEAM_E_UNSUPPORTED, "%s: unknown kv dtype %d", fn, kv->dtype);
  if (kv->dtype == BEAM_KV_FP8_E4M3 && !(kv->k_scale > 0.f && kv->v_scale > 0.f))
    return fail(BEAM_E_SHAPE, "%s: fp8 cache scales must be > 0", fn);
  if (kv->npos != 0 && kv->npos < kv->Lmax)
    return fail(BEAM_E_SHAPE, "%s: npos %d is neither 0 nor >= Lmax %d", fn, kv->npos, kv->Lmax);
  return BEAM_OK;
}
// Positions a cache accepts, and whether it is a ring (slot = position mod Lmax).
int kv_npos(const beam_kv* kv) { return kv->npos ? kv->npos : kv->Lmax; }
bool kv_ring(const beam_kv* kv) { return kv->npos > kv->Lmax; }
// Attention over a cache: max_pos below npos; a ring serves sliding-window
// attention only, with the window inside the ring.
int check_attn_cache(const beam_dims* dims, const beam_kv* kv, int swa, int max_pos,
                     const char* fn) {
  if (max_pos < 0 || max_pos >= kv_npos(kv))
    return fail(BEAM_E_SHAPE, "%s: max_pos %d outside [0, %d)", fn, max_pos, kv_npos(kv));
  if (kv_ring(kv) && !swa)
    return fail(BEAM_E_UNSUPPORTED, "%s: a ring cache serves sliding-window attention only", fn);
  if (kv_ring(kv) && dims->window > kv->Lmax)
    return fail(BEAM_E_SHAPE, "%s: window %d exceeds the ring's %d slots", fn, dims->window,
                kv->Lmax);
  return BEAM_OK;
}

// Every workspace is [kCtlBytes of counters][the call's data].
constexpr size_t kCtl = beam::kCtlBytes;
char* ws_data(void* ws) { return (char*)ws + kCtl; }
unsigned* ws_ctl(void* ws) { return (unsigned*)ws; }

size_t ws_qkv_payload(const beam_dims* d, int T) {
  return align256((size_t)T * (d->Hq + 2 * d->Hkv) * d->d * 2);
}
size_t ws_qkv(const beam_dims* d, int T) {
  return kCtl + ws_qkv_payload(d, T) +
         beam::gemm_split_bytes(T, (d->Hq + 2 * d->Hkv) * d->d + d->G, d->D);
}
int attn_span(const beam_dims* d, int swa, int max_ctx) {
  return swa ? std::min(max_ctx, d->window + 63) : max_ctx;
}
// Whether an attention call runs the flash kernel (else split-K per token).
// The workspace bound cannot see the cache's slot count, so it covers the
// split-K partials for every call of up to kDecodeBatchMaxT tokens.
bool attn_flash(const beam_dims* d, int T, int S) {
  if (T <= beam::kGemvMaxT || !beam::attn_prefill_ok(d->Hq / d->Hkv, d->d)) return false;
  return T > beam::kDecodeBatchMaxT || T > 4 * S;
}
size_t ws_attn(const beam_dims* d, int swa, int T, int max_ctx) {
  if (T > beam::kDecodeBatchMaxT && d->Hkv > 0 && beam::attn_prefill_ok(d->Hq / d->Hkv, d->d))
    return kCtl;  // the many-token kernel needs no partials
  const int nch = beam::attn_nch_bound(T, d->Hkv, attn_span(d, swa, max_ctx));
  if (nch == 1) return kCtl;
  return kCtl + align256((size_t)T * d->Hq * nch * (d->d + 4) * 4);
}
// One-token fused decode attention: [counters][raw q|k|v][gate][split-K
// records][normed q, for the long-context plan that runs the q/k epilogue in
// its own kernel], the records sized for the NoPE (full-context) span, which
// bounds the sliding-window one.
size_t ws_attn_fused(const beam_dims* d, int T, int max_ctx) {
  return ws_attn(d, 0, T, max_ctx) + ws_qkv_payload(d, T) +
         align256((size_t)T * d->G * 2) + align256((size_t)T * d->Hq * d->d * 2);
}
size_t ws_out_gate_payload(const beam_dims* d, int T) {
  return align256((size_t)T * d->Hq * d->d * 2);
}
size_t ws_out_gate(const beam_dims* d, int T) {
  return kCtl + ws_out_gate_payload(d, T) + beam::gemm_split_bytes(T, d->D, d->Hq * d->d);
}
// Router workspace: [counters][logits, when the caller passes none][K-split
// partial logits of the many-token GEMM, when it splits].
size_t ws_router_logits(const beam_dims* d, int T, bool own_logits) {
  return own_logits ? align256((size_t)T * d->E * 4) : 0;
}
size_t ws_router(const beam_dims* d, int T, bool own_logits = true) {
  size_t n = kCtl + ws_router_logits(d, T, own_logits);
  if (T > 4 && d->E > 0 && d->D > 0) {
    const int ns = beam::router_splits(T, d->E, d->D);
    if (ns > 1) n += align256((size_t)ns * T * d->E * 4);
  }
  return n;
}
float* ws_router_part(const beam_dims* d, int T, bool own_logits, void* ws) {
  return (float*)(ws_data(ws) + ws_router_logits(d, T, own_logits));
}

// Many-token MoE workspace, in order: counts[chunks][E+1], seg_off[E+2],
// tile_off[E+2], perm[P], inv[P] (int32); act[P][F] bf16; out[P][D] fp32, for
// P = T * (topk + 1) (token, slot) rows: a shared expert is routed as one more
// slot per token, segment E, through the same grouped GEMMs.
struct MoeWs {
  size_t counts, seg_off, tile_off, perm, inv, act, out, total;
};
MoeWs moe_ws_layout(const beam_dims* d, int T) {
  const size_t P = (size_t)T * (d->topk + 1), E = d->E;
  // chunk counts are not monotone in the pair count: room for either
  const size_t nch = std::max(beam::moe_route_chunks(T * d->topk),
                              beam::moe_route_chunks(T * (d->topk + 1)));
  MoeWs w{};
  size_t o = 0;
  w.counts = o; o += align256(nch * (E + 1) * 4);
  w.seg_off = o; o += align256((E + 2) * 4);
  w.tile_off = o; o += align256((E + 2) * 4);
  w.perm = o; o += align256(P * 4);
  w.inv = o; o += align256(P * 4);
  w.act = o; o += align256(P * d->F * 2);
  w.out = o; o += align256(P * d->D * 4);
  w.total = o;
  return w;
}
// Scaled-operand MoE: the pair -> row map, the MXFP8 copy of x, the
// activations (rows in expert order), then the other routing buffers, the
// MXFP8 copy of the activations and the per-pair outputs.
struct MoeMxWs {
  size_t counts, seg_off, tile_off, perm, inv, xq, xs, act, aq, as, out, total;
};
MoeMxWs moe_mx_ws_layout(const beam_dims* d, int T) {
  const size_t P = (size_t)T * d->topk, E = d->E, D = d->D, F = d->F;
  MoeMxWs w{};
  size_t o = 0;
  // the staged operands first (inv, xq, xs, act), at offsets a caller can
  // compute from T, topk, D and F alone
  w.inv = o; o += align256(P * 4);
  w.xq = o; o += align256((size_t)T * D);
  w.xs = o; o += align256((size_t)T * D / 32);
  w.act = o; o += align256(P * F * 2);
  w.counts = o; o += align256(beam::moe_route_chunks((int)P) * (E + 1) * 4);
  w.seg_off = o; o += align256((E + 2) * 4);
  w.tile_off = o; o += align256((E + 2) * 4);
  w.perm = o; o += align256(P * 4);
  w.aq = o; o += align256(P * F);
  w.as = o; o += align256(P * F / 32);
  w.out = o; o += align256(P * D * 4);
  w.total = o;
  return w;
}
bool moe_many(const beam_dims* d, int T) {
  return T > beam::kGemvMaxT && d->D % 64 == 0 && d->F % 64 == 0;
}
size_t ws_moe(const beam_dims* d, int T) {
  if (moe_many(d, T)) return kCtl + moe_ws_layout(d, T).total;
  return kCtl + align256((size_t)T * (d->topk + 1) * d->F * 2);
}
size_t ws_dense(int T, int Fd, int D) {
  return kCtl + align256((size_t)T * Fd * 2) +
         std::max(beam::gemm_split_bytes(T, 2 * Fd, D), beam::gemm_split_bytes(T, D, Fd));
}

int attn_impl(const beam_dims* dims, int T, const uint16_t* q, const int32_t* pos,
              const int32_t* seq, const beam_kv* kv, const float* sink, uint16_t* o,
              int max_pos, void* ws, size_t ws_bytes, void* stream, int swa, const char* fn,
              bool clear_ctl = false) {
  if (!dims) return fail(BEAM_E_NULL, "%s: dims is NULL", fn);
  if (!q || !pos || !seq || !o) return fail(BEAM_E_NULL, "%s: NULL tensor argument", fn);
  if (misaligned(q) || misaligned(o) || misaligned(ws) || misaligned(sink))
    return fail(BEAM_E_ALIGN, "%s: tensor not 16-byte aligned", fn);
  int rc = check_dims_attn(dims, fn);
  if (rc) return rc;
  if ((rc = check_kv(kv, fn))) return rc;
  if (T <= 0) return fail(BEAM_E_SHAPE, "%s: T <= 0", fn);
  if (swa && dims->window <= 0) return fail(BEAM_E_SHAPE, "%s: window <= 0", fn);
  if ((rc = check_attn_cache(dims, kv, swa, max_pos, fn))) return rc;
  const int fp8 = kv->dtype == BEAM_KV_FP8_E4M3;
  if (attn_flash(dims, T, kv->S)) {
    if (!ws || ws_bytes < kCtl)
      return fail(ws ? BEAM_E_WORKSPACE : BEAM_E_NULL, "%s: workspace %zu < %zu bytes", fn,
                  ws ? ws_bytes : 0, kCtl);
    if ((rc = device_ready())) return rc;
    if (clear_ctl && beam::launch_zero_words(ws_ctl(ws), (int)(kCtl / 4), S_(stream)))
      return launched(-1, fn);
    return launched(beam::launch_attn_prefill(T, dims->Hq, dims->Hkv, dims->d, swa, dims->window,
                                              fp8, q, pos, seq, kv->k, kv->v,
                                              fp8 ? kv->k_scale : 1.f, fp8 ? kv->v_scale : 1.f,
                                              kv->S, kv->Lmax, kv_npos(kv), sink, o,
                                              S_(stream)),
                    fn);
  }
  const int span = attn_span(dims, swa, max_pos + 1);
  const size_t need = ws_attn(dims, swa, T, max_pos + 1);
  if (!ws || ws_bytes < need)
    return fail(ws ? BEAM_E_WORKSPACE : BEAM_E_NULL, "%s: workspace %zu < %zu bytes", fn,
                ws ? ws_bytes : 0, need);
  if ((rc = device_ready())) return rc;
  if (clear_ctl && beam::launch_zero_words(ws_ctl(ws), (int)(kCtl / 4), S_(stream)))
    return launched(-1, fn);
  return launched(beam::launch_attn_decode(T, dims->Hq, dims->Hkv, dims->d, swa, dims->window,
                                           fp8, q, pos, seq, kv->k, kv->v,
                                           fp8 ? kv->k_scale : 1.f, fp8 ? kv->v_scale : 1.f,
                                           kv->S, kv->Lmax, kv_npos(kv), sink, o, span,
                                           (float*)ws_data(ws),
                                           ws_ctl(ws), S_(stream)),
                  fn);
}

// Argument checks of the router (shared by the fused boundary + router call).
int check_router(const beam_dims* dims, int T, const uint16_t* x, const float* w_r, int32_t* idx,
                 float* w, float* logits, void* ws, size_t ws_bytes, const char* fn) {
  if (!dims || !x || !w_r || !idx || !w) return fail(BEAM_E_NULL, "%s: NULL argument", fn);
  if (misaligned(x) || misaligned(w_r) || misaligned(logits) || misaligned(ws))
    return fail(BEAM_E_ALIGN, "%s: tensor not 16-byte aligned", fn);
  if (T <= 0) return fail(BEAM_E_SHAPE, "%s: T <= 0", fn);
  const int E = dims->E, ng = dims->n_group, tg = dims->topk_group, K = dims->topk;
  if (!(E > 0 && ng > 0 && tg > 0 && K > 0))
    return fail(BEAM_E_SHAPE, "%s: non-positive routing size", fn);
  if (E % ng) return fail(BEAM_E_SHAPE, "%s: E %% n_group != 0", fn);
  if (tg > ng) return fail(BEAM_E_SHAPE, "%s: topk_group > n_group", fn);
  if (K > tg * (E / ng)) return fail(BEAM_E_SHAPE, "%s: topk > topk_group * E / n_group", fn);
  if (K > 32) return fail(BEAM_E_UNSUPPORTED, "%s: topk > 32", fn);
  if (E > 1024 || ng > 64) return fail(BEAM_E_UNSUPPORTED, "%s: E > 1024 or n_group > 64", fn);
  if (!(dims->D > 0 && dims->D % 8 == 0))
    return fail(BEAM_E_UNSUPPORTED, "%s: D must be a positive multiple of 8", fn);
  if (!ws) return fail(BEAM_E_NULL, "%s: ws is NULL", fn);
  const size_t need = ws_router(dims, T, logits == nullptr);
  if (ws_bytes < need)
    return fail(BEAM_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  return BEAM_OK;
}

}  // namespace

namespace beam {

int abi_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int attn_entry(const beam_dims* dims, int T, const uint16_t* q, const int32_t* pos,
               const int32_t* seq, const beam_kv* kv, const float* sink, uint16_t* o,
               int max_pos, void* ws, size_t ws_bytes, void* stream, int swa, bool clear_ctl,
               const char* fn) {
  return attn_impl(dims, T, q, pos, seq, kv, sink, o, max_pos, ws, ws_bytes, stream, swa, fn,
                   clear_ctl);
}

}  // namespace beam

extern "C" {

int beam_version(void) { return BEAM_VERSION; }

const char* beam_last_error(void) { return g_last_error.c_str(); }

int beam_boundary_norm_residual(const beam_dims* dims, int T, const uint16_t* y,
                                const uint16_t* w_post, uint16_t* h, const uint16_t* w_pre,
                                uint16_t* x_out, int n, void* stream) {
  REQ(dims);
  REQ(h);
  REQ(w_pre);
  REQ(x_out);
  ALN(y);
  ALN(w_post);
  ALN(h);
  ALN(w_pre);
  ALN(x_out);
  SHAPE(T > 0, "%s: T <= 0", __func__);
  SHAPE(n >= 0, "%s: n < 0", __func__);
  UNSUP(dims->D > 0 && dims->D % 8 == 0 && dims->D <= 8192,
        "%s: D must be a positive multiple of 8 <= 8192", __func__);
  int rc = device_ready();
  if (rc) return rc;
  return launched(beam::launch_boundary(T, dims->D, y, w_post, h, w_pre, x_out, n, dims->eps,
                                        S_(stream)),
                  __func__);
}

int beam_qk_norm_rope_ssmax_kvwrite(const beam_dims* dims, int T, const uint16_t* x,
                                    const uint16_t* w_qkvg, const uint16_t* w_qnorm,
                                    const uint16_t* w_knorm, const int32_t* pos,
                                    const int32_t* seq, int mode, const float* rope_cs,
                                    uint16_t* q_out, uint16_t* g_out, const beam_kv* kv,
                                    void* ws, size_t ws_bytes, void* stream) {
  REQ(dims);
  REQ(x);
  REQ(w_qkvg);
  REQ(w_qnorm);
  REQ(w_knorm);
  REQ(pos);
  REQ(seq);
  REQ(q_out);
  REQ(ws);
  ALN(x);
  ALN(w_qkvg);
  ALN(q_out);
  ALN(g_out);
  ALN(ws);
  int rc = check_dims_attn(dims, __func__);
  if (rc) return rc;
  if ((rc = check_kv(kv, __func__))) return rc;
  SHAPE(T > 0, "%s: T <= 0", __func__);
  if (mode != BEAM_SWA_ROPE && mode != BEAM_NOPE_SSMAX)
    return fail(BEAM_E_SHAPE, "%s: invalid mode %d", __func__, mode);
  if (mode == BEAM_SWA_ROPE && !rope_cs)
    return fail(BEAM_E_NULL, "%s: RoPE mode needs rope_cs", __func__);
  if (mode == BEAM_NOPE_SSMAX && kv_ring(kv))
    return fail(BEAM_E_UNSUPPORTED, "%s: a ring cache serves sliding-window layers only",
                __func__);
  if (dims->G > 0 && !g_out) return fail(BEAM_E_NULL, "%s: g_out is NULL", __func__);
  if (ws_bytes < ws_qkv(dims, T))
    return fail(BEAM_E_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes,
                ws_qkv(dims, T));
  if ((rc = device_ready())) return rc;
  const int Nqkv = (dims->Hq + 2 * dims->Hkv) * dims->d;
  uint16_t* qkv = (uint16_t*)ws_data(ws);
  const int rcg = (T > beam::kGemvMaxT && dims->D % 64 == 0)
                      ? beam::launch_gemm_bf16(T, Nqkv + dims->G, dims->D, x, dims->D, w_qkvg,
                                               dims->D, qkv, Nqkv, g_out, dims->G, Nqkv,
                                               (float*)(ws_data(ws) + ws_qkv_payload(dims, T)),
                                               S_(stream))
                      : beam::launch_gemv_qkvg(T, Nqkv + dims->G, dims->D, Nqkv, w_qkvg, x, qkv,
                                               g_out, S_(stream));
  if (rcg) return launched(-1, __func__);
  const int fp8 = kv->dtype == BEAM_KV_FP8_E4M3;
  return launched(beam::launch_qk_epilogue(T, dims->Hq, dims->Hkv, dims->d, qkv, w_qnorm,
                                           w_knorm, pos, seq, mode, rope_cs, q_out, kv->k,
                                           kv->v, fp8, fp8 ? kv->k_scale : 1.f,
                                           fp8 ? kv->v_scale : 1.f, kv->S, kv->Lmax,
                                           kv_npos(kv), dims->eps, S_(stream)),
                  __func__);
}

int beam_attn_decode_fused(const beam_dims* dims, int T, const uint16_t* x,
                           const uint16_t* w_qkvg, const uint16_t* w_qnorm,
                           const uint16_t* w_knorm, const int32_t* pos, const int32_t* seq,
                           int mode, const float* rope_cs, const beam_kv* kv, const float* sink,
                           const uint16_t* b_gate, uint16_t* q_out, uint16_t* z_out, int max_pos,
                           void* ws, size_t ws_bytes, void* stream) {
  REQ(dims);
  REQ(x);
  REQ(w_qkvg);
  REQ(w_qnorm);
  REQ(w_knorm);
  REQ(pos);
  REQ(seq);
  REQ(z_out);
  REQ(ws);
  ALN(x);
  ALN(w_qkvg);
  ALN(q_out);
  ALN(z_out);
  ALN(ws);
  ALN(sink);
  int rc = check_dims_attn(dims, __func__);
  if (rc) return rc;
  if ((rc = check_kv(kv, __func__))) return rc;
  UNSUP(T == 1, "%s: one token per call (T = %d); use the separate calls for more", __func__, T);
  if (mode != BEAM_SWA_ROPE && mode != BEAM_NOPE_SSMAX)
    return fail(BEAM_E_SHAPE, "%s: invalid mode %d", __func__, mode);
  if (mode == BEAM_SWA_ROPE && !rope_cs)
    return fail(BEAM_E_NULL, "%s: RoPE mode needs rope_cs", __func__);
  if (mode == BEAM_SWA_ROPE && dims->window <= 0)
    return fail(BEAM_E_SHAPE, "%s: window <= 0", __func__);
  if (dims->G > 0 && !b_gate) return fail(BEAM_E_NULL, "%s: b_gate is NULL", __func__);
  if ((rc = check_attn_cache(dims, kv, mode == BEAM_SWA_ROPE, max_pos, __func__))) return rc;
  const size_t need = ws_attn_fused(dims, T, max_pos + 1);
  if (ws_bytes < need)
    return fail(BEAM_E_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes, need);
  if ((rc = device_ready())) return rc;
  const int swa = mode == BEAM_SWA_ROPE;
  const int Nqkv = (dims->Hq + 2 * dims->Hkv) * dims->d;
  uint16_t* qkv = (uint16_t*)ws_data(ws);
  uint16_t* gbuf = (uint16_t*)(ws_data(ws) + ws_qkv_payload(dims, T));
  float* part = (float*)(ws_data(ws) + ws_qkv_payload(dims, T) +
                         align256((size_t)T * dims->G * 2));
  if (beam::launch_gemv_qkvg(T, Nqkv + dims->G, dims->D, Nqkv, w_qkvg, x, qkv, gbuf, S_(stream)))
    return launched(-1, __func__);
  const int fp8 = kv->dtype == BEAM_KV_FP8_E4M3;
  const float ks = fp8 ? kv->k_scale : 1.f, vs = fp8 ? kv->v_scale : 1.f;
  const int span = attn_span(dims, swa, max_pos + 1);
  beam::AttnFuse fz{qkv, w_qnorm, w_knorm, rope_cs, dims->eps, swa ? 0 : 1, ks, vs,
                    dims->G > 0 ? gbuf : nullptr, dims->G > 0 ? b_gate : nullptr, q_out};
  // A long fp8 context streams through thousands of split-K workgroups with a
  // separate merge; fused, each of them would first form q from the raw
  // projection, a start-up repeated for every round of resident workgroups.
  // There the q/k epilogue (with the cache write) runs once in its own kernel
  // and only the gate stays fused, into the merge.
  int tpw, nch;
  beam::attn_plan(T, dims->Hkv, span, &tpw, &nch);
  const uint16_t* q_in = nullptr;
  if (fp8 && nch > 1 && !beam::attn_fused_merge(T, dims->Hkv, nch)) {
    uint16_t* qn = q_out ? q_out
                         : (uint16_t*)((char*)part + (ws_attn(dims, 0, T, max_pos + 1) - kCtl));
    if (beam::launch_qk_epilogue(T, dims->Hq, dims->Hkv, dims->d, qkv, w_qnorm, w_knorm, pos,
                                 seq, swa ? 0 : 1, rope_cs, qn, kv->k, kv->v, fp8, ks, vs, kv->S,
                                 kv->Lmax, kv_npos(kv), dims->eps, S_(stream)))
      return launched(-1, __func__);
    q_in = qn;
    fz.qkv = nullptr;
  }
  return launched(beam::launch_attn_decode(T, dims->Hq, dims->Hkv, dims->d, swa, dims->window,
                                           fp8, q_in, pos, seq, kv->k, kv->v, ks, vs, kv->S,
                                           kv->Lmax, kv_npos(kv), sink, z_out, span, part,
                                           ws_ctl(ws), S_(stream), &fz),
                  __func__);
}

int beam_attn_swa(const beam_dims* dims, int T, const uint16_t* q, const int32_t* pos,
                  const int32_t* seq, const beam_kv* kv, const float* sink, uint16_t* o,
                  int max_pos, void* ws, size_t ws_bytes, void* stream) {
  return attn_impl(dims, T, q, pos, seq, kv, sink, o, max_pos, ws, ws_bytes, stream, 1,
                   __func__);
}

int beam_attn_nope_ssmax(const beam_dims* dims, int T, const uint16_t* q,
                         const int32_t* pos, const int32_t* seq, const beam_kv* kv,
                         const float* sink, uint16_t* o, int max_pos, void* ws,
                         size_t ws_bytes, void* stream) {
  return attn_impl(dims, T, q, pos, seq, kv, sink, o, max_pos, ws, ws_bytes, stream, 0,
                   __func__);
}

int beam_out_gate(const beam_dims* dims, int T, const uint16_t* o, const uint16_t* g,
                  const uint16_t* b_gate, const uint16_t* w_o, uint16_t* y, void* ws,
                  size_t ws_bytes, void* stream) {
  REQ(dims);
  REQ(o);
  REQ(w_o);
  REQ(y);
  ALN(o);
  ALN(g);
  ALN(w_o);
  ALN(y);
  ALN(ws);
  int rc = check_dims_attn(dims, __func__);
  if (rc) return rc;
  SHAPE(T > 0, "%s: T <= 0", __func__);
  if (g && !b_gate) return fail(BEAM_E_NULL, "%s: gate bias is NULL", __func__);
  const bool gate = dims->G > 0 && g != nullptr;
  const int K = dims->Hq * dims->d;
  if (T > beam::kGemvMaxT && K % 64 == 0) {
    const uint16_t* a = o;
    if (gate) {
      REQ(ws);
      if (ws_bytes < ws_out_gate(dims, T))
        return fail(BEAM_E_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes,
                    ws_out_gate(dims, T));
    }
    // split-K partials when the workspace holds them (a batch of decode steps)
    float* part = (ws && ws_bytes >= ws_out_gate(dims, T))
                      ? (float*)(ws_data(ws) + ws_out_gate_payload(dims, T))
                      : nullptr;
    if ((rc = device_ready())) return rc;
    if (gate) {
      if (beam::launch_gate(T, dims->Hq, dims->d, o, g, b_gate, (uint16_t*)ws_data(ws),
                            S_(stream)))
        return launched(-1, __func__);
      a = (const uint16_t*)ws_data(ws);
    }
    return launched(beam::launch_gemm_bf16(T, dims->D, K, a, K, w_o, K, y, dims->D, nullptr, 0,
                                           dims->D, part, S_(stream)),
                    __func__);
  }
  if ((rc = device_ready())) return rc;
  return launched(beam::launch_gemv_gate_oproj(T, dims->D, K, dims->d, w_o, o,
                                               gate ? g : nullptr, b_gate, y, S_(stream)),
                  __func__);
}


int beam_router_fp32_grouped_topk(const beam_dims* dims, int T, const uint16_t* x,
                                  const float* w_r, const float* b_corr, int32_t* idx,
                                  float* w, float* logits, void* ws, size_t ws_bytes,
                                  void* stream) {
  int rc = check_router(dims, T, x, w_r, idx, w, logits, ws, ws_bytes, __func__);
  if (rc) return rc;
  float* lg = logits ? logits : (float*)ws_data(ws);
  if ((rc = device_ready())) return rc;
  return launched(beam::launch_router(T, dims->E, dims->D, dims->n_group, dims->topk_group,
                                      dims->topk, dims->route_scale, x, w_r, b_corr, lg, idx, w,
                                      ws_router_part(dims, T, logits == nullptr, ws), ws_ctl(ws),
                                      S_(stream)),
                  __func__);
}

int beam_boundary_router_fp32_grouped_topk(const beam_dims* dims, int T, const uint16_t* y,
                                           const uint16_t* w_post, uint16_t* h,
                                           const uint16_t* w_pre, uint16_t* x_out, int n,
                                           const float* w_r, const float* b_corr,
                                           int32_t* idx, float* w, float* logits, void* ws,
                                           size_t ws_bytes, void* stream) {
  REQ(dims);
  REQ(h);
  REQ(w_pre);
  ALN(y);
  ALN(w_post);
  ALN(h);
  ALN(w_pre);
  SHAPE(n >= 0, "%s: n < 0", __func__);
  UNSUP(dims->D > 0 && dims->D % 8 == 0 && dims->D <= 8192,
        "%s: D must be a positive multiple of 8 <= 8192", __func__);
  int rc = check_router(dims, T, x_out, w_r, idx, w, logits, ws, ws_bytes, __func__);
  if (rc) return rc;
  float* lg = logits ? logits : (float*)ws_data(ws);
  if ((rc = device_ready())) return rc;
  return launched(beam::launch_boundary_router(T, dims->D, y, w_post, h, w_pre, x_out, n,
                                               dims->eps, dims->E, dims->n_group,
                                               dims->topk_group, dims->topk, dims->route_scale,
                                               w_r, b_corr, lg, idx, w,
                                               ws_router_part(dims, T, logits == nullptr, ws),
                                               ws_ctl(ws), S_(stream)),
                  __func__);
}

namespace {
// shared by the MXFP8 and MXFP4 entry points (bits = 8 or 4 per weight)
int mx_quantize(int bits, const uint16_t* w, size_t rows, int K, uint8_t* codes,
                uint8_t* scales, void* stream, const char* fn) {
  if (!w || !codes || !scales) return fail(BEAM_E_NULL, "%s: NULL tensor argument", fn);
  if (misaligned(w) || misaligned(codes))
    return fail(BEAM_E_ALIGN, "%s: tensor not 16-byte aligned", fn);
  if (K <= 0 || K % 32) return fail(BEAM_E_SHAPE, "%s: K must be a positive multiple of 32", fn);
  if (rows == 0) return BEAM_OK;
  const int rc = device_ready();
  if (rc) return rc;
  const long long nb = (long long)rows * (K / 32);
  return launched(bits == 8 ? beam::launch_mxfp8_quantize(w, nb, codes, scales, S_(stream))
                            : beam::launch_mxfp4_quantize(w, nb, codes, scales, S_(stream)),
                  fn);
}

int moe_mx(int bits, const beam_dims* dims, int T, const uint16_t* x, const int32_t* idx,
           const float* w, const uint8_t* w13_codes, const uint8_t* w13_scales,
           const uint8_t* w2_codes, const uint8_t* w2_scales, uint16_t* y, void* ws,
           size_t ws_bytes, void* stream, const char* fn) {
  if (!dims) return fail(BEAM_E_NULL, "%s: dims is NULL", fn);
  if (!x || !idx || !w || !w13_codes || !w13_scales || !w2_codes || !w2_scales || !y || !ws)
    return fail(BEAM_E_NULL, "%s: NULL tensor argument", fn);
  if (misaligned(x) || misaligned(w13_codes) || misaligned(w2_codes) || misaligned(y) ||
      misaligned(ws))
    return fail(BEAM_E_ALIGN, "%s: tensor not 16-byte aligned", fn);
  if (T <= 0) return fail(BEAM_E_SHAPE, "%s: T <= 0", fn);
  if (dims->E <= 0 || dims->topk <= 0 || dims->F <= 0)
    return fail(BEAM_E_SHAPE, "%s: non-positive E/topk/F", fn);
  if (T > beam::kGemvMaxT)
    return fail(BEAM_E_UNSUPPORTED, "%s: block-scaled experts are decode-only (T <= %d)", fn,
                beam::kGemvMaxT);
  if (!(dims->D > 0 && dims->D % 32 == 0 && dims->D <= 5120))
    return fail(BEAM_E_UNSUPPORTED, "%s: D must be a positive multiple of 32 <= 5120", fn);
  if (!(dims->F % 32 == 0 && dims->F <= 2560))
    return fail(BEAM_E_UNSUPPORTED, "%s: F must be a multiple of 32 <= 2560", fn);
  const size_t need = kCtl + align256((size_t)T * dims->topk * dims->F * 2);
  if (ws_bytes < need)
    return fail(BEAM_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  const int rc = device_ready();
  if (rc) return rc;
  uint16_t* act = (uint16_t*)ws_data(ws);
  const hipStream_t st = S_(stream);
  const int D = dims->D, F = dims->F, E = dims->E, K = dims->topk;
  return launched(bits == 8 ? beam::launch_moe_mxfp8(T, D, F, E, K, w13_codes, w13_scales,
                                                     w2_codes, w2_scales, idx, w, x, act, y, st)
                            : beam::launch_moe_mxfp4(T, D, F, E, K, w13_codes, w13_scales,
                                                     w2_codes, w2_scales, idx, w, x, act, y, st),
                  fn);
}
}  // namespace

int beam_mxfp8_quantize(const uint16_t* w, size_t rows, int K, uint8_t* codes, uint8_t* scales,
                        void* stream) {
  return mx_quantize(8, w, rows, K, codes, scales, stream, __func__);
}

int beam_mxfp4_quantize(const uint16_t* w, size_t rows, int K, uint8_t* codes, uint8_t* scales,
                        void* stream) {
  return mx_quantize(4, w, rows, K, codes, scales, stream, __func__);
}

int beam_moe_swiglu_combine_mxfp8(const beam_dims* dims, int T, const uint16_t* x,
                                  const int32_t* idx, const float* w, const uint8_t* w13_codes,
                                  const uint8_t* w13_scales, const uint8_t* w2_codes,
                                  const uint8_t* w2_scales, uint16_t* y, void* ws,
                                  size_t ws_bytes, void* stream) {
  return moe_mx(8, dims, T, x, idx, w, w13_codes, w13_scales, w2_codes, w2_scales, y, ws,
                ws_bytes, stream, __func__);
}

int beam_moe_swiglu_combine_mxfp4(const beam_dims* dims, int T, const uint16_t* x,
                                  const int32_t* idx, const float* w, const uint8_t* w13_codes,
                                  const uint8_t* w13_scales, const uint8_t* w2_codes,
                                  const uint8_t* w2_scales, uint16_t* y, void* ws,
                                  size_t ws_bytes, void* stream) {
  return moe_mx(4, dims, T, x, idx, w, w13_codes, w13_scales, w2_codes, w2_scales, y, ws,
                ws_bytes, stream, __func__);
}

int beam_moe_swiglu_combine_mx_scaled(const beam_dims* dims, int T, const uint16_t* x,
                                      const int32_t* idx, const float* w, int wbits,
                                      const uint8_t* w13_codes, const uint8_t* w13_scales,
                                      const uint8_t* w2_codes, const uint8_t* w2_scales,
                                      uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  REQ(dims);
  REQ(x);
  REQ(idx);
  REQ(w);
  REQ(w13_codes);
  REQ(w13_scales);
  REQ(w2_codes);
  REQ(w2_scales);
  REQ(y);
  REQ(ws);
  ALN(x);
  ALN(w13_codes);
  ALN(w2_codes);
  ALN(y);
  ALN(ws);
  if (((uintptr_t)w13_scales | (uintptr_t)w2_scales) & 3)
    return fail(BEAM_E_ALIGN, "%s: scales not 4-byte aligned", __func__);
  SHAPE(T > 0, "%s: T <= 0", __func__);
  SHAPE(wbits == 8 || wbits == 4, "%s: weight format %d is neither 8 (MXFP8) nor 4 (MXFP4)",
        __func__, wbits);
  SHAPE(dims->E > 0 && dims->E <= 1024 && dims->topk > 0 && dims->F > 0,
        "%s: E must be in [1, 1024], topk and F positive", __func__);
  UNSUP(dims->D % 128 == 0 && dims->F % 128 == 0,
        "%s: D and F must be multiples of 128 (the slab depth)", __func__);
  const size_t need = kCtl + moe_mx_ws_layout(dims, T).total;
  if (ws_bytes < need)
    return fail(BEAM_E_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes, need);
  int rc = device_ready();
  if (rc) return rc;
  const MoeMxWs L = moe_mx_ws_layout(dims, T);
  char* b = ws_data(ws);
  int32_t* counts = (int32_t*)(b + L.counts);
  int32_t* seg_off = (int32_t*)(b + L.seg_off);
  int32_t* tile_off = (int32_t*)(b + L.tile_off);
  int32_t* perm = (int32_t*)(b + L.perm);
  int32_t* inv = (int32_t*)(b + L.inv);
  uint8_t* xq = (uint8_t*)(b + L.xq);
  uint8_t* xs = (uint8_t*)(b + L.xs);
  uint16_t* act = (uint16_t*)(b + L.act);
  uint8_t* aq = (uint8_t*)(b + L.aq);
  uint8_t* as = (uint8_t*)(b + L.as);
  float* out = (float*)(b + L.out);
  const int E = dims->E, K = dims->topk, D = dims->D, F = dims->F;
  const int P = T * K;
  const int BMr = beam::gemm_mx_rows();
  const int max_tiles = (P + BMr - 1) / BMr + E;
  const bool b4 = wbits == 4;
  const hipStream_t st = S_(stream);
  // route; x -> MXFP8; gate/up with SwiGLU; act -> MXFP8; down; combine
  if (beam::launch_moe_route(T, K, K, E, idx, BMr, counts, seg_off, tile_off, perm, inv, st) ||
      beam::launch_mxfp8_quantize(x, (long long)T * D / 32, xq, xs, st) ||
      beam::launch_gemm_mx_swiglu(F, D, xq, xs, perm, w13_codes, w13_scales, b4, seg_off,
                                  tile_off, E, max_tiles, act, st) ||
      beam::launch_mxfp8_quantize(act, (long long)P * F / 32, aq, as, st) ||
      beam::launch_gemm_mx_f32(D, F, aq, as, w2_codes, w2_scales, b4, seg_off, tile_off, E,
                               max_tiles, out, st))
    return launched(-1, __func__);
  return launched(beam::launch_moe_combine(T, K, K, E, D, out, inv, w, idx, y, st), __func__);
}

int beam_moe_swiglu_combine(const beam_dims* dims, int T, const uint16_t* x,
                            const int32_t* idx, const float* w, const uint16_t* w13,
                            const uint16_t* w2, const uint16_t* shared_w13,
                            const uint16_t* shared_w2, uint16_t* y, void* ws,
                            size_t ws_bytes, void* stream) {
  REQ(dims);
  REQ(x);
  REQ(idx);
  REQ(w);
  REQ(w13);
  REQ(w2);
  REQ(y);
  REQ(ws);
  ALN(x);
  ALN(w13);
  ALN(w2);
  ALN(shared_w13);
  ALN(shared_w2);
  ALN(y);
  ALN(ws);
  SHAPE(T > 0, "%s: T <= 0", __func__);
  SHAPE(dims->E > 0 && dims->topk > 0 && dims->F > 0, "%s: non-positive E/topk/F", __func__);
  if ((shared_w13 == nullptr) != (shared_w2 == nullptr))
    return fail(BEAM_E_NULL, "%s: shared_w13 and shared_w2 must both be set or both NULL",
                __func__);
  UNSUP(dims->D > 0 && dims->D % 8 == 0 && dims->D <= 8192,
        "%s: D must be a positive multiple of 8 <= 8192", __func__);
  UNSUP(dims->F % 8 == 0, "%s: F must be a multiple of 8", __func__);
  if (ws_bytes < ws_moe(dims, T))
    return fail(BEAM_E_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes,
                ws_moe(dims, T));
  int rc = device_ready();
  if (rc) return rc;
  if (moe_many(dims, T)) {
    const MoeWs L = moe_ws_layout(dims, T);
    char* b = ws_data(ws);
    int32_t* counts = (int32_t*)(b + L.counts);
    int32_t* seg_off = (int32_t*)(b + L.seg_off);
    int32_t* tile_off = (int32_t*)(b + L.tile_off);
    int32_t* perm = (int32_t*)(b + L.perm);
    int32_t* inv = (int32_t*)(b + L.inv);
    uint16_t* act = (uint16_t*)(b + L.act);
    float* out = (float*)(b + L.out);
    const int E = dims->E, K = dims->topk, D = dims->D, F = dims->F;
    // a shared expert is one more slot per token (segment E, weight 1) in the
    // same routing permutation and grouped GEMMs as the routed experts
    const int spt = K + (shared_w13 ? 1 : 0), NE = E + (shared_w13 ? 1 : 0);
    const int P = T * spt;
    const int BMr = beam::gemm_grouped_rows(P, NE);
    const int max_tiles = (P + BMr - 1) / BMr + NE;
    const hipStream_t st = S_(stream);
    if (beam::launch_moe_route(T, K, spt, E, idx, BMr, counts, seg_off, tile_off, perm, inv,
                               st) ||
        beam::launch_gemm_swiglu(P, F, D, x, D, perm, w13, seg_off, tile_off, NE,
                                 (long long)2 * F * D, max_tiles, act, nullptr, st, shared_w13) ||
        beam::launch_gemm_f32(P, D, F, act, F, w2, seg_off, tile_off, NE, (long long)D * F,
                              max_tiles, out, D, st, shared_w2))
      return launched(-1, __func__);
    return launched(beam::launch_moe_combine(T, K, spt, E, D, out, inv, w, idx, y, st),
                    __func__);
  }
  const int spt = dims->topk + (shared_w13 ? 1 : 0);
  uint16_t* act = (uint16_t*)ws_data(ws);
  if (beam::launch_expert_w13(T, dims->D, dims->F, dims->E, dims->topk, spt, w13, shared_w13,
                              idx, x, act, S_(stream)))
    return launched(-1, __func__);
  return launched(beam::launch_expert_w2(T, dims->D, dims->F, dims->E, dims->topk, spt, w2,
                                         shared_w2, idx, w, act, y, S_(stream)),
                  __func__);
}

int beam_moe_experts_up(const beam_dims* dims, int T, const uint16_t* x, const int32_t* idx,
                        const uint16_t* w13, const uint16_t* shared_w13, uint16_t* act,
                        void* stream) {
  REQ(dims);
  REQ(x);
  REQ(idx);
  REQ(w13);
  REQ(act);
  ALN(x);
  ALN(w13);
  ALN(shared_w13);
  ALN(act);
  SHAPE(T > 0, "%s: T <= 0", __func__);
  SHAPE(dims->E > 0 && dims->topk > 0 && dims->F > 0, "%s: non-positive E/topk/F", __func__);
  UNSUP(dims->D > 0 && dims->D % 8 == 0 && dims->D <= 8192,
        "%s: D must be a positive multiple of 8 <= 8192", __func__);
  UNSUP(dims->F % 8 == 0, "%s: F must be a multiple of 8", __func__);
  int rc = device_ready();
  if (rc) return rc;
  const int spt = dims->topk + (shared_w13 ? 1 : 0);
  return launched(beam::launch_expert_w13(T, dims->D, dims->F, dims->E, dims->topk, spt, w13,
                                          shared_w13, idx, x, act, S_(stream)),
                  __func__);
}

int beam_moe_experts_down(const beam_dims* dims, int T, const int32_t* idx, const float* w,
                          const uint16_t* w2, const uint16_t* shared_w2, const uint16_t* act,
                          uint16_t* y, void* stream) {
  REQ(dims);
  REQ(idx);
  REQ(w);
  REQ(w2);
  REQ(act);
  REQ(y);
  ALN(w2);
  ALN(shared_w2);
  ALN(act);
  ALN(y);
  SHAPE(T > 0, "%s: T <= 0", __func__);
  SHAPE(dims->E > 0 && dims->topk > 0 && dims->F > 0, "%s: non-positive E/topk/F", __func__);
  UNSUP(dims->D > 0 && dims->D % 8 == 0 && dims->D <= 8192,
        "%s: D must be a positive multiple of 8 <= 8192", __func__);
  UNSUP(dims->F % 8 == 0, "%s: F must be a multiple of 8", __func__);
  int rc = device_ready();
  if (rc) return rc;
  const int spt = dims->topk + (shared_w2 ? 1 : 0);
  return launched(beam::launch_expert_w2(T, dims->D, dims->F, dims->E, dims->topk, spt, w2,
                                         shared_w2, idx, w, act, y, S_(stream)),
                  __func__);
}

int beam_dense_swiglu(int T, int D, int Fd, const uint16_t* x, const uint16_t* w13,
                      const uint16_t* w2, uint16_t* y, void* ws, size_t ws_bytes,
                      void* stream) {
  REQ(x);
  REQ(w13);
  REQ(w2);
  REQ(y);
  REQ(ws);
  ALN(x);
  ALN(w13);
  ALN(w2);
  ALN(y);
  ALN(ws);
  SHAPE(T > 0, "%s: T <= 0", __func__);
  SHAPE(Fd > 0 && Fd % 64 == 0, "%s: Fd must be a positive multiple of 64", __func__);
  UNSUP(D > 0 && D % 8 == 0 && D <= 8192, "%s: D must be a positive multiple of 8 <= 8192",
        __func__);
  if (ws_bytes < ws_dense(T, Fd, D))
    return fail(BEAM_E_WORKSPACE, "%s: workspace %zu < %zu bytes", __func__, ws_bytes,
                ws_dense(T, Fd, D));
  int rc = device_ready();
  if (rc) return rc;
  uint16_t* act = (uint16_t*)ws_data(ws);
  if (T > beam::kGemvMaxT && D % 64 == 0) {
    float* part = (float*)(ws_data(ws) + align256((size_t)T * Fd * 2));
    if (beam::launch_gemm_swiglu(T, Fd, D, x, D, nullptr, w13, nullptr, nullptr, 1, 0, 0, act,
                                 part, S_(stream)))
      return launched(-1, __func__);
    return launched(beam::launch_gemm_bf16(T, D, Fd, act, Fd, w2, Fd, y, D, nullptr, 0, D, part,
                                           S_(stream)),
                    __func__);
  }
  if (beam::launch_expert_w13(T, D, Fd, 1, 1, 1, w13, nullptr, nullptr, x, act, S_(stream)))
    return launched(-1, __func__);
  return launched(beam::launch_expert_w2(T, D, Fd, 1, 1, 1, w2, nullptr, nullptr, nullptr, act,
                                         y, S_(stream)),
                  __func__);
}

int beam_lm_head_softcap(int T, int D, int V, const uint16_t* x, const uint16_t* w, float cap,
                         float* logits, void* stream) {
  REQ(x);
  REQ(w);
  REQ(logits);
  ALN(x);
  ALN(w);
  ALN(logits);
  SHAPE(T > 0 && V > 0, "%s: T or V <= 0", __func__);
  SHAPE(cap >= 0.f && cap <= 3.0e38f, "%s: cap must be finite and >= 0", __func__);
  UNSUP(D > 0 && D % 8 == 0 && D <= 8192, "%s: D must be a positive multiple of 8 <= 8192",
        __func__);
  const int rc = device_ready();
  if (rc) return rc;
  const hipStream_t st = S_(stream);
  if (T > beam::kGemvMaxT && D % 64 == 0) {
    if (beam::launch_gemm_f32(T, V, D, x, D, w, nullptr, nullptr, 1, 0, 0, logits, V, st))
      return launched(-1, __func__);
    if (cap == 0.f) return BEAM_OK;
    return launched(beam::launch_softcap(logits, (long long)T * V, cap, st), __func__);
  }
  return launched(beam::launch_gemv_lm_head(T, V, D, w, x, cap, logits, st), __func__);
}

size_t beam_workspace_size(const beam_dims* dims, int op, int T, int max_ctx) {
  if (!dims || T <= 0) return (size_t)-1;
  switch (op) {
    case BEAM_OP_QKV: return ws_qkv(dims, T);
    case BEAM_OP_ATTN_SWA:
    case BEAM_OP_ATTN_NOPE:
      if (max_ctx <= 0 || dims->Hkv <= 0) return (size_t)-1;
      return ws_attn(dims, op == BEAM_OP_ATTN_SWA, T, max_ctx);
    case BEAM_OP_OUT_GATE: return ws_out_gate(dims, T);
    case BEAM_OP_ROUTER: return ws_router(dims, T);
    case BEAM_OP_MOE: return ws_moe(dims, T);
    case BEAM_OP_DENSE: return ws_dense(T, dims->F, dims->D);
    case BEAM_OP_MOE_MX_SCALED:
      if (dims->D <= 0 || dims->F <= 0 || dims->topk <= 0 || dims->E <= 0) return (size_t)-1;
      return kCtl + moe_mx_ws_layout(dims, T).total;
    case BEAM_OP_ATTN_DECODE_FUSED:
      if (max_ctx <= 0 || dims->Hkv <= 0) return (size_t)-1;
      return ws_attn_fused(dims, T, max_ctx);
    default: return (size_t)-1;
  }
}

int beam_hbm_read(const void* p, size_t bytes, unsigned* sink, void* stream) {
  REQ(p);
  REQ(sink);
  ALN(p);
  SHAPE(bytes % 16 == 0, "%s: bytes must be a multiple of 16", __func__);
  int rc = device_ready();
  if (rc) return rc;
  return launched(beam::launch_hbm_read(p, bytes, sink, S_(stream)), __func__);
}

int beam_rope_table(float* out, int Lmax, int d, double theta) {
  if (!out) return fail(BEAM_E_NULL, "%s: out is NULL", __func__);
  if (Lmax <= 0 || d <= 0 || d % 2 || !(theta > 0))
    return fail(BEAM_E_SHAPE, "%s: bad Lmax/d/theta", __func__);
  const int half = d / 2;
  for (int i = 0; i < half; ++i) {
    const double inv_freq = std::pow(theta, -2.0 * i / d);
    for (int p = 0; p < Lmax; ++p) {
      const double a = (double)p * inv_freq;
      out[(size_t)p * d + i] = (float)std::cos(a);
      out[(size_t)p * d + half + i] = (float)std::sin(a);
    }
  }
  return BEAM_OK;
}

int beam_check(void* stream) {
  int rc = device_ready();
  if (rc) return rc;
  hipError_t e = hipStreamSynchronize(S_(stream));
  if (e != hipSuccess) return fail(BEAM_E_HIP, "beam_check: %s", hipGetErrorString(e));
  const int f = beam::gemv_read_clear_err() | beam::qk_read_clear_err() |
                beam::attn_read_clear_err() | beam::attnp_read_clear_err() |
                beam::moe_read_clear_err() |
                beam::mx_read_clear_err();
  if (f < 0) return fail(BEAM_E_HIP, "beam_check: reading the device flags failed");
  if (f)
    return fail(BEAM_E_DEVICE, "beam_check: device check tripped:%s%s%s%s%s",
                (f & 1) ? " position outside the cache" : "",
                (f & 2) ? " sequence slot outside the cache" : "",
                (f & 4) ? " expert id outside [0, E)" : "",
                (f & 8) ? " position beyond the call's max_pos" : "",
                (f & 16) ? " value outside the fp16 range of the attention product" : "");
  return BEAM_OK;
}

}  // extern "C"
