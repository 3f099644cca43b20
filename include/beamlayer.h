/*
 * libbeamlayer — forward pass of one Beam-style sparse MoE decoder layer on
 * AMD MI355X (gfx950), at batch-1 decode and at chunked prefill.
 *
 * What the layer computes is described on the "Reflection Beam 1.0 on vLLM"
 * page (sections cited per call as [Attn], [MoE], [Opt]):
 *   [Attn] "Attention: sliding-window layers and NoPE full-attention layers"
 *   [MoE]  "MoE and residual stream: FP32 router, sandwich norm, depth-scaled residual"
 *   [Opt]  "Agent-driven optimisation makes batch-1 decode 2.71x faster"
 *          (its seven numbered changes are cited as [Opt]/1 .. [Opt]/7)
 *   [Graph] "The fused decode graph runs one MoE layer in 13 kernels"
 * and, for the second model's variant switches, the "vLLM Day-0 support:
 * Recursive's Flint" page, section "Flint model architecture" [Flint].
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Types: bf16 tensors are passed as uint16_t bit patterns, fp8 e4m3fn (OCP)
 *    cache entries as uint8_t codes, router tensors as float (binary32),
 *    token positions, sequence slots and expert ids as int32_t.
 *  - Memory: every tensor argument is a caller-owned DEVICE pointer, row-major,
 *    contiguous and 16-byte aligned. Structs (beam_dims, beam_kv) live in host
 *    memory; their pointer fields are device pointers. The library allocates
 *    nothing: calls that need scratch take a caller-owned device workspace
 *    (`ws`, `ws_bytes`), sized by beam_workspace_size(). A workspace starts
 *    with a 1024-byte block of counters (used where the last workgroup to
 *    finish combines the others' partial results) that must hold zeros when a
 *    call starts; every call that completes leaves it zeroed, so zero-fill a
 *    workspace once when it is allocated (and again after a device fault).
 *    The rest of its contents is ignored on entry and undefined on exit. One
 *    workspace may serve every call that is ordered on one stream.
 *  - Streams: `stream` is a hipStream_t (NULL = the null stream). Every call
 *    only enqueues kernels on it: no host synchronisation, no allocation, no
 *    memset, so every call may be captured into a HIP graph. Inputs must not
 *    be modified until the enqueued work completes.
 *  - Status: every call returns BEAM_OK (0) or a negative BEAM_E_* code.
 *    Arguments are validated on the host before any HIP call (NULL pointers,
 *    shapes, alignment, workspace size); then the device is checked
 *    (BEAM_E_NODEV when no GPU is present); launch failures give BEAM_E_HIP.
 *    beam_last_error() returns a thread-local message for the last failure.
 *  - Data-dependent checks run on the device: a position outside the cache,
 *    a position beyond the max_pos an attention call was given, or an expert
 *    id outside [0, E) skips the offending token or expert (an attention
 *    output row it leaves is written as zeros) and raises a device error flag
 *    that beam_check() reports; so does a value the many-token attention
 *    kernel had to clamp to the fp16 range of its P.V operand.
 *  - Threading: calls are reentrant; two calls that share output buffers or a
 *    workspace must be ordered by the caller (same stream).
 *
 * KV-cache layout (one cache per layer, caller-owned):
 *  - K: [S][Hkv][Lmax][d]  (key-major: one key's d values contiguous)
 *  - V: [S][Hkv][d][Lmax]  (value-transposed: one dim's values over positions
 *                           contiguous), so that the attention contraction over
 *                           keys reads contiguous runs for the matrix cores.
 *  - Element type bf16, or fp8 e4m3fn codes c with value decode(c) * scale
 *    (one k_scale for the whole K cache, one v_scale for V).
 *  - Lmax must be a multiple of 64. The index over Lmax is a slot: the
 *    position itself, or the position mod Lmax in a ring (beam_kv.npos).
 */
#ifndef BEAMLAYER_H
#define BEAMLAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BEAM_VERSION 100

enum beam_status {
  BEAM_OK = 0,
  BEAM_E_NULL = -1,        /* a required pointer is NULL                         */
  BEAM_E_SHAPE = -2,       /* inconsistent or out-of-range sizes                 */
  BEAM_E_UNSUPPORTED = -3, /* sizes outside the compiled specialisations, dtype  */
  BEAM_E_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned            */
  BEAM_E_WORKSPACE = -5,   /* ws_bytes smaller than beam_workspace_size()        */
  BEAM_E_HIP = -6,         /* a HIP launch or runtime call failed                */
  BEAM_E_NODEV = -7,       /* no usable GPU                                      */
  BEAM_E_DEVICE = -8       /* a device-side check tripped (see beam_check)       */
};

enum beam_attn_mode { BEAM_SWA_ROPE = 0, BEAM_NOPE_SSMAX = 1 };
enum beam_kv_dtype { BEAM_KV_BF16 = 0, BEAM_KV_FP8_E4M3 = 1 };
enum beam_op {
  BEAM_OP_QKV = 1,       /* beam_qk_norm_rope_ssmax_kvwrite */
  BEAM_OP_ATTN_SWA = 2,  /* beam_attn_swa                   */
  BEAM_OP_ATTN_NOPE = 3, /* beam_attn_nope_ssmax            */
  BEAM_OP_OUT_GATE = 4,  /* beam_out_gate                   */
  BEAM_OP_ROUTER = 5,    /* beam_router_fp32_grouped_topk   */
  BEAM_OP_MOE = 6,       /* beam_moe_swiglu_combine         */
  BEAM_OP_DENSE = 7,     /* beam_dense_swiglu (dims->F read as the dense d_ff) */
  BEAM_OP_ATTN_DECODE_FUSED = 8, /* beam_attn_decode_fused                  */
  BEAM_OP_MOE_MX_SCALED = 9      /* beam_moe_swiglu_combine_mx_scaled       */
};

/* Layer shape. D hidden size; Hq/Hkv query/kv heads (Hq % Hkv == 0, group
 * Hq/Hkv <= 16); d head dim (32, 64 or 128); G gate width (Hq*d: one gate
 * value per attention output element, or 0 for no output gate); E experts in
 * n_group groups, keep topk_group groups then topk experts; F expert d_ff;
 * window SWA keys including the current token; eps RMSNorm epsilon;
 * route_scale multiplier of the renormalised routing weights (2.5 on Beam). */
typedef struct beam_dims {
  int D, Hq, Hkv, d, G, E, n_group, topk_group, topk, F, window;
  float eps, route_scale;
} beam_dims;

/* One layer's KV cache (see the layout above). k, v: device pointers;
 * dtype: beam_kv_dtype; k_scale/v_scale: fp8 dequantisation scales (> 0,
 * ignored for bf16); S sequence slots; Lmax slots per sequence (a multiple
 * of 64); npos the positions the cache accepts: 0 (or Lmax) for one slot per
 * position, positions [0, Lmax); a value above Lmax makes each sequence's
 * slots a ring: position p lives in slot p mod Lmax and positions [0, npos)
 * are accepted ([Attn]: a sliding-window layer keeps only its last `window`
 * keys). A ring serves sliding-window attention only (calls in mode
 * BEAM_NOPE_SSMAX reject it) and needs window <= Lmax; within one call the
 * keys each token reads must still be in the ring after the call's own cache
 * writes, i.e. Lmax >= window + (tokens of one sequence in the call) - 1 (not
 * checked: a smaller ring silently reads newer keys in place of old ones).
 * The RoPE table passed with a cache has a row for every accepted position. */
typedef struct beam_kv {
  void* k;
  void* v;
  int dtype;
  float k_scale, v_scale;
  int S, Lmax;
  int npos;
} beam_kv;

/* Sublayer boundary [MoE] sandwich norm + depth-scaled residual, fused as in
 * [Opt]/1:   a = RMSNorm(y; w_post)                (bf16)
 *            h <- sqrt((n-1)/n) * h + a / sqrt(n)  (bf16, in place)
 *            x_out = RMSNorm(h; w_pre)             (bf16)
 * RMSNorm(v; w) = v / sqrt(mean(v^2) + eps) * w, statistics in fp32.
 * y [T][D], h [T][D] (in/out), x_out [T][D], gains [D], all bf16.
 * y == NULL: only x_out = RMSNorm(h; w_pre) (the layer-entry pre-norm; h is
 * read only). w_post == NULL: a = y (no post-norm). n == 0: plain add h + a
 * (pre-norm models, [Flint]). Errors: T <= 0, D not a multiple of 8 or
 * above 8192, n < 0. */
int beam_boundary_norm_residual(const beam_dims* dims, int T, const uint16_t* y,
                                const uint16_t* w_post, uint16_t* h,
                                const uint16_t* w_pre, uint16_t* x_out, int n,
                                void* stream);

/* Packed projection and per-head Q/K processing with the cache write
 * ([Opt]/5 packed q|k|v|gate GEMM, [Opt]/2 and [Opt]/6 fused norm, RoPE/SSMax
 * and KV update; [Attn]):
 *   qkvg = bf16(x . w_qkvg^T), w_qkvg [Hq*d + 2*Hkv*d + G][D] bf16 with row
 *   blocks q (head-major), k, v, gate.
 *   q_h <- RMSNorm_d(q_h; w_qnorm), k_j <- RMSNorm_d(k_j; w_knorm) (one [d]
 *   gain each, shared by all heads), then
 *     mode BEAM_SWA_ROPE:   rotate q and k at position pos[t] (rotate-half
 *                           pairs (i, i+d/2); rope_cs[pos][i] = cos, and
 *                           rope_cs[pos][d/2+i] = sin, of pos*theta^(-2i/d),
 *                           table [npos][d] fp32, see beam_rope_table);
 *     mode BEAM_NOPE_SSMAX: q <- q * (1 + (pos[t]+1)/2048)^0.1, keys as is.
 *   q_out [T][Hq][d] = bf16(q); g_out [T][G] = the gate rows (bf16);
 *   cache slot (seq[t], pos[t]) <- k, v (bf16, or e4m3 of value/scale with
 *   round-to-nearest-even and saturation at 448).
 * x [T][D] bf16; pos, seq [T] int32 (device). ws >= beam_workspace_size(QKV).
 * Errors: invalid mode; RoPE without rope_cs; Hq % Hkv; d unsupported; fp8
 * with a scale <= 0. Device check: pos outside [0, npos) or seq outside
 * [0, S) skips that token's cache write and raises the device flag. */
int beam_qk_norm_rope_ssmax_kvwrite(const beam_dims* dims, int T, const uint16_t* x,
                                    const uint16_t* w_qkvg, const uint16_t* w_qnorm,
                                    const uint16_t* w_knorm, const int32_t* pos,
                                    const int32_t* seq, int mode, const float* rope_cs,
                                    uint16_t* q_out, uint16_t* g_out, const beam_kv* kv,
                                    void* ws, size_t ws_bytes, void* stream);

/* GQA attention over a sliding window [Attn]: query head h of token t reads
 * kv head floor(h*Hkv/Hq) of slot seq[t] at positions
 * [max(0, pos[t]-window+1), pos[t]] (window keys including itself), scores
 * q.k/sqrt(d), fp32 softmax and accumulation, o [T][Hq][d] bf16.
 * sink (optional, [Flint]): per-head fp32 logit added to the softmax
 * denominator only. max_pos >= max(pos) (host value used to size the grid
 * and the split-K records; a token beyond it is not attended: its output row
 * is zero and the device flag is raised).
 * ws >= beam_workspace_size(ATTN_SWA, T, max_pos + 1) (counter block and
 * split-K partials).
 * Kernels: calls of T <= 4 tokens, and of T <= 256 tokens with T <= 4 * kv->S
 * (a batch of decode steps over many sequences), run split-K per token; other
 * calls (prefill chunks) run a flash kernel that shares each key tile among
 * the tokens of a sequence. Both compute the same function; they differ in the
 * precision of the P.V product: split-K kernels carry each probability to ~16
 * bits (a bf16 hi + lo pair), the flash kernel on a bf16 cache with d = 128
 * rounds probabilities to fp16 and converts V to fp16 (exact for bf16 values
 * of magnitude <= 65504; larger ones are clamped to +-65504 and the device
 * flag is raised, so beam_check reports BEAM_E_DEVICE for such a call; an
 * infinite or NaN cached value among the keys a call reads raises it too).
 * Errors: window <= 0, max_pos >= npos; a ring cache with window > Lmax. */
int beam_attn_swa(const beam_dims* dims, int T, const uint16_t* q, const int32_t* pos,
                  const int32_t* seq, const beam_kv* kv, const float* sink, uint16_t* o,
                  int max_pos, void* ws, size_t ws_bytes, void* stream);

/* Full-context attention of a NoPE layer [Attn]: as beam_attn_swa over all
 * positions [0, pos[t]]; the SSMax query scale was applied by the q/k call.
 * ws >= beam_workspace_size(ATTN_NOPE, T, max_pos + 1) (split-K partials). */
int beam_attn_nope_ssmax(const beam_dims* dims, int T, const uint16_t* q,
                         const int32_t* pos, const int32_t* seq, const beam_kv* kv,
                         const float* sink, uint16_t* o, int max_pos, void* ws,
                         size_t ws_bytes, void* stream);

/* One-token fused attention half for batch-1 decode ([Opt] changes 2, 5 and
 * 6; [FlintOpt] low-latency path: q/k norm, RoPE and the KV write fused into
 * the kernels next to them): the packed projection, then ONE attention
 * kernel that applies the per-head q/k RMSNorm with RoPE (mode
 * BEAM_SWA_ROPE) or the SSMax query scale (BEAM_NOPE_SSMAX) to the raw
 * projection, writes the new k and v to the cache at (seq[0], pos[0]),
 * attends (the sliding window or the full context, as beam_attn_swa /
 * beam_attn_nope_ssmax) and, when dims->G > 0, applies the output gate at
 * its merge:
 *   z_out [1][Hq*d] = bf16(bf16(o) * sigmoid(g + b_gate[head]))   (G > 0)
 *                   = o                                          (G == 0)
 * so that beam_out_gate(..., g = NULL, ...) then runs o_proj on z_out alone.
 * Results are those of beam_qk_norm_rope_ssmax_kvwrite, the attention call
 * and the gate of beam_out_gate composed (same arithmetic). q_out
 * (nullable) receives the normed q [1][Hq][d]. T must be 1 (otherwise
 * BEAM_E_UNSUPPORTED). ws >= beam_workspace_size(ATTN_DECODE_FUSED, 1,
 * max_pos + 1), counter block zeroed once. Errors as the three calls. */
int beam_attn_decode_fused(const beam_dims* dims, int T, const uint16_t* x,
                           const uint16_t* w_qkvg, const uint16_t* w_qnorm,
                           const uint16_t* w_knorm, const int32_t* pos, const int32_t* seq,
                           int mode, const float* rope_cs, const beam_kv* kv, const float* sink,
                           const uint16_t* b_gate, uint16_t* q_out, uint16_t* z_out, int max_pos,
                           void* ws, size_t ws_bytes, void* stream);

/* Allocation-free beam_attn_nope_ssmax, for callers that cannot allocate or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, results and errors as
 * beam_attn_nope_ssmax without ws / ws_bytes: the split-K records and
 * counters live in a static device array of 16 MiB per GPU (held by each GPU
 * the library runs on until the process ends); its counter block is cleared
 * by a kernel on `stream` at the start of every call. Calls whose workspace
 * need (beam_workspace_size(ATTN_NOPE, T, max_pos + 1)) exceeds 16 MiB are
 * rejected with BEAM_E_WORKSPACE before anything is launched. At the Beam
 * shape (48 query / 8 kv heads of 128) one to four tokens fit at contexts up
 * to 8M positions, a batch of 128 decode steps up to 81,920 positions, 256
 * steps up to 32,768; many-token chunks (flash kernel) need the counters only.
 * The call allocates nothing. Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (different streams, or threads) race and must
 * be ordered by the caller. */
int beam_attn_nope_ssmax_static(const beam_dims* dims, int T, const uint16_t* q,
                                const int32_t* pos, const int32_t* seq, const beam_kv* kv,
                                const float* sink, uint16_t* o, int max_pos, void* stream);

/* Sigmoid output gate and o_proj ([Attn]; [Opt]/2 gate kernel):
 *   z = bf16(o * sigmoid(g + b_gate[head]))  elementwise over [T][Hq*d]
 *   y = bf16(z . w_o^T), w_o [D][Hq*d] bf16, y [T][D] bf16.
 * g == NULL: z = o, o_proj alone (a layer without a gate, G == 0, or an input
 * the gate was already applied to, e.g. by beam_attn_decode_fused).
 * ws >= beam_workspace_size(OUT_GATE).
 * Errors: G not in {0, Hq*d}; b_gate NULL while g is given. */
int beam_out_gate(const beam_dims* dims, int T, const uint16_t* o, const uint16_t* g,
                  const uint16_t* b_gate, const uint16_t* w_o, uint16_t* y, void* ws,
                  size_t ws_bytes, void* stream);

/* FP32 router with DeepSeek-V3 grouped selection ([MoE]; [Opt]/4):
 *   logits = fp32(x) . w_r^T (fp32 weights [E][D], fp32 accumulation)
 *   s = sigmoid(logits); s' = s + b_corr (b_corr may be NULL = 0)
 *   group score = sum of the two largest s' in each of n_group groups;
 *   keep topk_group groups; pick topk experts by s' among them;
 *   w = route_scale * s / sum(s) over the picked experts.
 * Ties go to the lower index; idx [T][topk] int32 ordered by s' descending,
 * w [T][topk] fp32, logits [T][E] fp32 (optional output).
 * ws >= beam_workspace_size(ROUTER): the counter block, the logits when the
 * caller passes none, and for T > 4 the partial logits of the K-split GEMM
 * (when few token tiles split D; T * E * 4 bytes per split, at most D/128
 * splits). With T <= 4 and logits given, 1024 bytes suffice.
 * Errors: E % n_group; topk_group > n_group; topk > topk_group*E/n_group;
 * topk > 32; E > 1024. */
int beam_router_fp32_grouped_topk(const beam_dims* dims, int T, const uint16_t* x,
                                  const float* w_r, const float* b_corr, int32_t* idx,
                                  float* w, float* logits, void* ws, size_t ws_bytes,
                                  void* stream);

/* The attention-side boundary followed by the router, as one call:
 * exactly beam_boundary_norm_residual(dims, T, y, w_post, h, w_pre, x_out, n)
 * then beam_router_fp32_grouped_topk(dims, T, x_out, w_r, b_corr, idx, w,
 * logits, ws, ws_bytes) ([MoE]; [Opt]/1 and /4), same results bit for bit.
 * At T = 1 it runs as one kernel: every router workgroup computes the
 * boundary row while its expert rows load and uses it as the GEMV input, and
 * the last workgroup stores h and x_out. Arguments and errors are those of the
 * two calls; ws as for the router. */
int beam_boundary_router_fp32_grouped_topk(const beam_dims* dims, int T, const uint16_t* y,
                                           const uint16_t* w_post, uint16_t* h,
                                           const uint16_t* w_pre, uint16_t* x_out, int n,
                                           const float* w_r, const float* b_corr,
                                           int32_t* idx, float* w, float* logits, void* ws,
                                           size_t ws_bytes, void* stream);

/* Routed SwiGLU experts and the weighted combine ([MoE]; [Opt]/3 combine):
 *   for each token t and k < topk, e = idx[t][k]:
 *     u = bf16(x_t . w13[e]^T)   w13 [E][2F][D] bf16 (rows 0..F-1 gate, F..2F-1 up)
 *     a = bf16(silu(u[:F]) * u[F:])
 *     acc += w[t][k] * (a . w2[e]^T)  (fp32)   w2 [E][D][F] bf16
 *   plus, when shared_w13 != NULL, one always-on expert with weight 1 ([Flint]);
 *   y [T][D] = bf16(acc).
 * Only the selected experts' weights are read. ws >= beam_workspace_size(MOE).
 * Device check: ids outside [0, E) are skipped and raise the device flag. */
int beam_moe_swiglu_combine(const beam_dims* dims, int T, const uint16_t* x,
                            const int32_t* idx, const float* w, const uint16_t* w13,
                            const uint16_t* w2, const uint16_t* shared_w13,
                            const uint16_t* shared_w2, uint16_t* y, void* ws,
                            size_t ws_bytes, void* stream);

/* The two phases of beam_moe_swiglu_combine, for callers that schedule them
 * separately (beam_moe_swiglu_combine == up, then down, with act in ws):
 *   up:   act[t][k][:] = bf16(silu(u[:F]) * u[F:]) for every routed slot k
 *         (and slot topk for the shared expert when shared_w13 != NULL);
 *         act [T][topk (+1)][F] bf16, caller-owned.
 *   down: y = bf16(sum_k w[t][k] * (act[t][k] . w2[e]^T) (+ shared, weight 1)).
 * Both read only the selected experts' rows. Device check as above. */
int beam_moe_experts_up(const beam_dims* dims, int T, const uint16_t* x, const int32_t* idx,
                        const uint16_t* w13, const uint16_t* shared_w13, uint16_t* act,
                        void* stream);
int beam_moe_experts_down(const beam_dims* dims, int T, const int32_t* idx, const float* w,
                          const uint16_t* w2, const uint16_t* shared_w2, const uint16_t* act,
                          uint16_t* y, void* stream);

/* Block-scaled FP8 experts (MXFP8). The pages run the routed experts in a
 * 4-bit block format ([MoE]: d_ff 2,560 "NVFP4"); this is the 8-bit member of
 * the OCP microscaling family: a weight row [K] is stored as K e4m3fn codes
 * (uint8) and K/32 E8M0 scale bytes, block b = elements [32b, 32b + 32) of
 * the row, value(code) * 2^(scale - 127). The shared exponent of a block is
 * floor(log2(max |w|)) - 8 (so max |w| / 2^exp lies in [256, 512)), each code
 * is w / 2^exp rounded to nearest even and saturated at +-448; an all-zero
 * block has scale byte 0.
 *
 * beam_mxfp8_quantize: w [rows][K] bf16 (device) -> codes [rows][K] and
 * scales [rows][K/32] (device). Errors: K not a positive multiple of 32. */
int beam_mxfp8_quantize(const uint16_t* w, size_t rows, int K, uint8_t* codes, uint8_t* scales,
                        void* stream);

/* beam_moe_swiglu_combine with MXFP8 expert weights, decode steps (T <= 4):
 * w13_codes [E][2F][D] (gate rows, then up rows) with w13_scales
 * [E][2F][D/32]; w2_codes [E][D][F] with w2_scales [E][D][F/32]. Maths as
 * beam_moe_swiglu_combine with every weight replaced by its dequantised value
 * (dot products in fp32; act and y rounded to bf16 at the same points); no
 * shared expert. Only the selected experts' codes and scales are read.
 * ws >= 1024 + T * topk * F * 2 bytes (beam_workspace_size(MOE) suffices).
 * Errors: T > 4 (UNSUPPORTED); D or F not a multiple of 32, D > 5120,
 * F > 2560. Expert ids outside [0, E) are skipped and flagged on the device. */
int beam_moe_swiglu_combine_mxfp8(const beam_dims* dims, int T, const uint16_t* x,
                                  const int32_t* idx, const float* w, const uint8_t* w13_codes,
                                  const uint8_t* w13_scales, const uint8_t* w2_codes,
                                  const uint8_t* w2_scales, uint16_t* y, void* ws,
                                  size_t ws_bytes, void* stream);

/* MXFP4: the same scheme with e2m1 elements (1 sign bit, 2 exponent bits with
 * bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), the format
 * family of the pages' 4-bit experts ([MoE]). Shared exponent of a block =
 * floor(log2(max |w|)) - 2 (max |w| / 2^exp in [4, 8)); codes round to nearest
 * even and saturate at +-6; two codes per byte, element 2i in the low nibble.
 *
 * beam_mxfp4_quantize: w [rows][K] bf16 (device) -> codes [rows][K/2] and
 * scales [rows][K/32] (device). Errors: K not a positive multiple of 32. */
int beam_mxfp4_quantize(const uint16_t* w, size_t rows, int K, uint8_t* codes, uint8_t* scales,
                        void* stream);

/* beam_moe_swiglu_combine_mxfp8 with MXFP4 expert weights: w13_codes
 * [E][2F][D/2], w13_scales [E][2F][D/32], w2_codes [E][D][F/2], w2_scales
 * [E][D][F/32]. Same maths, sizes, workspace and errors. */
int beam_moe_swiglu_combine_mxfp4(const beam_dims* dims, int T, const uint16_t* x,
                                  const int32_t* idx, const float* w, const uint8_t* w13_codes,
                                  const uint8_t* w13_scales, const uint8_t* w2_codes,
                                  const uint8_t* w2_scales, uint16_t* y, void* ws,
                                  size_t ws_bytes, void* stream);

/* Routed experts of a many-token step on block-scaled operands on both sides
 * of the products ([MoE]: experts in a 4-bit block format; [Opt]: the
 * library MoE path quantises the activations and runs two grouped GEMMs),
 * on gfx950's scaled matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4):
 *   xq = MXFP8(x)         each token row in blocks of 32 along D (e4m3 codes,
 *                         one E8M0 scale: floor(log2(amax)) - 8, RNE, saturating
 *                         at 448; the weights' rule)
 *   gate, up = bf16(xq . W13_e^T) (fp32 accumulation), act = bf16(silu(gate) * up)
 *   aq = MXFP8(act)       in blocks of 32 along F
 *   y = bf16(sum_k w[t][k] * (aq . W2_e^T))
 * with W13_e, W2_e the decoded block-scaled weights: wbits 8 (MXFP8: codes
 * w13 [E][2F][D], w2 [E][D][F]) or 4 (MXFP4: codes w13 [E][2F][D/2], w2
 * [E][D][F/2]); scales w13 [E][2F][D/32], w2 [E][D][F/32] (4-byte aligned),
 * as beam_mxfp8_quantize / beam_mxfp4_quantize write them. The activation
 * quantisation makes this a different function from beam_moe_swiglu_combine
 * on the decoded weights (each product input carries up to half an e4m3 step
 * of its block). Rows are routed as in beam_moe_swiglu_combine (tile rows
 * 256; ids outside [0, E) flagged and left out). T >= 1, D and F multiples
 * of 128, E <= 1024, no shared expert.
 * ws >= beam_workspace_size(BEAM_OP_MOE_MX_SCALED, T). After the call the
 * workspace's data area (past its 1 KiB counter block) starts with the staged
 * operands, each at a 256-byte-aligned offset, for inspection: the routed row
 * of each (token, slot) pair (int32 [T][topk]), xq's codes [T][D] and scales
 * [T][D/32], and the activations act (bf16 [T*topk][F], rows in expert order).
 * Errors: wbits not 8 or 4, sizes as above. */
int beam_moe_swiglu_combine_mx_scaled(const beam_dims* dims, int T, const uint16_t* x,
                                      const int32_t* idx, const float* w, int wbits,
                                      const uint8_t* w13_codes, const uint8_t* w13_scales,
                                      const uint8_t* w2_codes, const uint8_t* w2_scales,
                                      uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/* Output head with the logit soft cap (after the layer stack; Beam's
 * architecture notes give logits = 30 * tanh(z / 30)): x [T][D] bf16 (the
 * final normed hidden rows), w [V][D] bf16 (the head's rows), logits [T][V]
 * fp32 (device) = cap * tanh((x[t] . w[v]) / cap), or the plain dot product
 * when cap is 0. Dot products in fp32. T <= 4: weight-streaming GEMV with the
 * cap in its epilogue; larger T (D a multiple of 64): the matrix-core GEMM
 * into logits, then the cap in place. No workspace.
 * Errors: T or V <= 0 or cap negative / not finite (SHAPE); D not a positive
 * multiple of 8 <= 8,192 (UNSUPPORTED). */
int beam_lm_head_softcap(int T, int D, int V, const uint16_t* x, const uint16_t* w, float cap,
                         float* logits, void* stream);

/* Dense SwiGLU MLP of the first layers ([MoE]; [Opt]/7):
 *   u = bf16(x . w13^T) (w13 [2*Fd][D], gate rows then up rows),
 *   a = bf16(silu(u[:Fd]) * u[Fd:]), y = bf16(a . w2^T) (w2 [D][Fd]).
 * Errors: Fd % 64, D % 8. ws >= beam_workspace_size(DENSE) with dims->F = Fd. */
int beam_dense_swiglu(int T, int D, int Fd, const uint16_t* x, const uint16_t* w13,
                      const uint16_t* w2, uint16_t* y, void* ws, size_t ws_bytes,
                      void* stream);

/* Bytes of workspace `op` needs for T tokens; max_ctx bounds the attended
 * context (max_pos + 1) for the attention ops and is ignored otherwise.
 * Returns 0 for ops that need none and (size_t)-1 for invalid arguments. */
size_t beam_workspace_size(const beam_dims* dims, int op, int T, int max_ctx);

/* The Beam model's layer schedule ("Reflection Beam 1.0 on vLLM": model
 * architecture, Attention, MoE and residual stream sections): layer (0-based)
 * of an n_layers stack attends the full context without positions
 * (BEAM_NOPE_SSMAX) when its 1-based number is a multiple of 6 or it is the
 * last layer, else a sliding window with RoPE (BEAM_SWA_ROPE); layers 0-2 run
 * a dense SwiGLU FFN (*dense = 1), the others MoE. Of 52 layers: 43 + 9, and
 * 3 dense + 49 MoE. Errors: NULL outputs, layer outside [0, n_layers). */
int beam_layer_kind(int layer, int n_layers, int* attn_mode, int* dense);

/* One layer of a decode stack: attention mode (BEAM_SWA_ROPE or
 * BEAM_NOPE_SSMAX), FFN kind (dense 1: w13 [2 Fd][D] and w2 [D][Fd] of the
 * dense SwiGLU; dense 0: experts w13 [E][2F][D], w2 [E][D][F] and the fp32
 * router w_r [E][D], b_corr [E]), the sandwich norm gains, the attention
 * weights of the single-layer calls (device pointers) and the layer's KV cache
 * (a ring on sliding-window layers, see beam_kv). */
typedef struct beam_stack_layer {
  int attn_mode;
  int dense;
  const uint16_t *w_attn_pre, *w_attn_post, *w_ffn_pre, *w_ffn_post;
  const uint16_t *w_qnorm, *w_knorm, *w_qkvg, *b_gate, *w_o;
  const float *w_r, *b_corr;
  const uint16_t *w13, *w2;
  beam_kv kv;
} beam_stack_layer;

/* Workspace bytes of beam_decode_stack (counter block first; zero it once). */
size_t beam_decode_stack_workspace(const beam_dims* dims, int Fd, int max_ctx);

/* One decode step of one token through n_layers consecutive layers of a
 * sandwich-norm stack (the layer as the single-layer calls compose it, the
 * attention half through beam_attn_decode_fused), layers[0] being layer
 * `layer0` of the model:
 *   x = RMSNorm(h; layers[0].w_attn_pre)
 *   for each layer l (model index L = layer0 + l):
 *     z = attention half of x (cache write at pos); y = z . w_o^T
 *     h, x2 = boundary(y; w_attn_post, w_ffn_pre; residual add 2L + 1)
 *             (MoE layers: with the router's grouped top-k)
 *     y2 = MoE(x2) or dense SwiGLU(x2)
 *     h, x = boundary(y2; w_ffn_post, w_next; residual add 2L + 2),
 *            w_next = the next layer's w_attn_pre, or w_final after the last
 *   x_out = x (the output head's input when the run ends the model).
 * h [1][D] bf16 in/out; x_out [1][D]; pos, seq [1] int32 (device); rope_cs
 * the RoPE table of the sliding-window layers (a row per position up to
 * max_pos); max_pos >= pos[0]; Fd the dense d_ff (0 when no layer is dense).
 * dims describes every layer (dims->F the expert d_ff). Launches 6 calls per
 * layer on `stream`, so a whole step can be captured in one HIP graph.
 * ws >= beam_decode_stack_workspace(dims, Fd, max_pos + 1).
 * Errors: those of the composed calls (the first failing one), plus NULL
 * arguments, an invalid mode, a dense layer with Fd = 0, an MoE layer
 * without router weights. */
int beam_decode_stack(const beam_dims* dims, int Fd, int layer0, int n_layers,
                      const beam_stack_layer* layers, const uint16_t* w_final, uint16_t* h,
                      uint16_t* x_out, const int32_t* pos, const int32_t* seq,
                      const float* rope_cs, int max_pos, void* ws, size_t ws_bytes,
                      void* stream);

/* Host helper: fill out[Lmax][d] (host memory) with the RoPE table used by
 * beam_qk_norm_rope_ssmax_kvwrite, computed in double and stored as float. */
int beam_rope_table(float* out, int Lmax, int d, double theta);

/* Measurement utility (not part of the layer): reads `bytes` of device memory
 * at p once, with 16-byte non-temporal loads spread over the whole GPU, and
 * writes nothing but (at most) one word to the device word *sink. Timing it
 * gives a measured HBM streaming-read ceiling. bytes % 16 == 0, p 16-byte
 * aligned. */
int beam_hbm_read(const void* p, size_t bytes, unsigned* sink, void* stream);

/* Waits for `stream`, then reports BEAM_E_HIP for a failed kernel or
 * BEAM_E_DEVICE if a device-side check tripped since the last beam_check
 * (the flag is cleared). */
int beam_check(void* stream);

const char* beam_last_error(void);
int beam_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BEAMLAYER_H */
