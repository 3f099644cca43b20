// Host-side launchers of the libbeamlayer kernels (internal interface between
// the C ABI in abi.cpp and the kernel translation units). Each launcher only
// enqueues work on `st` and returns 0, or -1 when a launch fails.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "beamlayer.h"

namespace beam {

// Sets the thread-local message beam_last_error() returns; returns code.
int abi_fail(int code, const char* fmt, ...);
// The attention call behind beam_attn_swa / beam_attn_nope_ssmax (swa 1 / 0),
// with every argument check; clear_ctl zeroes the workspace's counter block
// (after the checks, on the call's stream) before the attention kernels run.
int attn_entry(const beam_dims* dims, int T, const uint16_t* q, const int32_t* pos,
               const int32_t* seq, const beam_kv* kv, const float* sink, uint16_t* o,
               int max_pos, void* ws, size_t ws_bytes, void* stream, int swa, bool clear_ctl,
               const char* fn);
int launch_zero_words(unsigned* p, int n, hipStream_t st);

int launch_boundary(int T, int D, const uint16_t* y, const uint16_t* w_post, uint16_t* h,
                    const uint16_t* w_pre, uint16_t* x_out, int n, float eps, hipStream_t st);

int launch_gemv_qkvg(int T, int N, int K, int Nqkv, const uint16_t* W, const uint16_t* X,
                     uint16_t* qkv, uint16_t* g_out, hipStream_t st);
int launch_gemv_gate_oproj(int T, int N, int K, int hd, const uint16_t* W, const uint16_t* O,
                           const uint16_t* G, const uint16_t* bgate, uint16_t* Y,
                           hipStream_t st);
// output head with the logit soft cap (cap 0: plain logits)
int launch_gemv_lm_head(int T, int V, int K, const uint16_t* W, const uint16_t* X, float cap,
                        float* logits, hipStream_t st);
int launch_softcap(float* z, long long n, float cap, hipStream_t st);
int launch_expert_w13(int T, int D, int F, int E, int topk, int spt, const uint16_t* w13,
                      const uint16_t* shared_w13, const int32_t* idx, const uint16_t* X,
                      uint16_t* act, hipStream_t st);
// block-scaled fp8 (MXFP8) experts, decode steps
int launch_mxfp8_quantize(const uint16_t* w, long long nblocks, uint8_t* codes, uint8_t* scales,
                          hipStream_t st);
int launch_moe_mxfp8(int T, int D, int F, int E, int topk, const uint8_t* w13c,
                     const uint8_t* w13s, const uint8_t* w2c, const uint8_t* w2s,
                     const int32_t* idx, const float* wts, const uint16_t* X, uint16_t* act,
                     uint16_t* Y, hipStream_t st);
// block-scaled operands on both sides (MXFP8 activations; MXFP8 or MXFP4
// weights), grouped expert GEMMs of many-token steps on the scaled matrix
// cores; K % 128 == 0, tile rows gemm_mx_rows()
int gemm_mx_rows();
int launch_gemm_mx_swiglu(int F, int K, const uint8_t* A, const uint8_t* As,
                          const int32_t* gather, const uint8_t* B, const uint8_t* Bs, bool b4,
                          const int32_t* seg_off, const int32_t* tile_off, int E,
                          int max_mtiles, uint16_t* act, hipStream_t st);
int launch_gemm_mx_f32(int N, int K, const uint8_t* A, const uint8_t* As, const uint8_t* B,
                       const uint8_t* Bs, bool b4, const int32_t* seg_off,
                       const int32_t* tile_off, int E, int max_mtiles, float* out,
                       hipStream_t st);

// block-scaled fp4 (MXFP4) experts, decode steps
int launch_mxfp4_quantize(const uint16_t* w, long long nblocks, uint8_t* codes, uint8_t* scales,
                          hipStream_t st);
int launch_moe_mxfp4(int T, int D, int F, int E, int topk, const uint8_t* w13c,
                     const uint8_t* w13s, const uint8_t* w2c, const uint8_t* w2s,
                     const int32_t* idx, const float* wts, const uint16_t* X, uint16_t* act,
                     uint16_t* Y, hipStream_t st);
int launch_expert_w2(int T, int D, int F, int E, int topk, int spt, const uint16_t* w2,
                     const uint16_t* shared_w2, const int32_t* idx, const float* wts,
                     const uint16_t* act, uint16_t* Y, hipStream_t st);

int launch_qk_epilogue(int T, int Hq, int Hkv, int hd, const uint16_t* qkv, const uint16_t* wq,
                       const uint16_t* wk, const int32_t* pos, const int32_t* seq, int mode,
                       const float* rope_cs, uint16_t* q_out, void* kc, void* vc, int fp8,
                       float k_scale, float v_scale, int S, int Lmax, int npos, float eps,
                       hipStream_t st);

// Every workspace starts with a block of kCtlBytes of zeroed uint32 counters
// (last-arriver elections); kernels that use them leave them at zero.
constexpr size_t kCtlBytes = 1024;
constexpr int kAttnCounters = 256;      // (token, kv head) pairs with a fused merge
constexpr int kAttnFusedMergeMax = 8;   // chunks the last workgroup still merges

// The decode attention kernel's fused mode (one token): the projection's
// epilogue (per-head q/k norm, RoPE or SSMax, the KV write) runs inside the
// attention kernel on the raw q|k|v rows, and the output gate at its merge.
struct AttnFuse {
  const uint16_t* qkv;    // raw projection [T][(Hq + 2 Hkv) * d], or null when q is given
                          // (then only the gate below is fused, into a separate merge)
  const uint16_t* wq;     // q / k norm gains [d]
  const uint16_t* wk;
  const float* rope;      // RoPE table [Lmax][d] (mode 0), else unused
  float eps;
  int mode;               // 0 RoPE (sliding window), 1 SSMax (NoPE)
  float ks, vs;           // fp8 cache scales (1 for bf16)
  const uint16_t* g;      // gate projection [T][Hq * d] and per-head bias, or null
  const uint16_t* bgate;
  uint16_t* q_out;        // normed q [T][Hq][d], or null
};

void attn_plan(int T, int Hkv, int span, int* tpw, int* nch);
int attn_nch_bound(int T, int Hkv, int span);
bool attn_fused_merge(int T, int Hkv, int nch);
int launch_attn_decode(int T, int Hq, int Hkv, int hd, int swa, int window, int fp8,
                       const uint16_t* q, const int32_t* pos, const int32_t* seq,
                       const void* kc, const void* vc, float k_scale, float v_scale, int S,
                       int Lmax, int npos, const float* sink, uint16_t* o, int span,
                       float* part, unsigned* ctr, hipStream_t st,
                       const AttnFuse* fuse = nullptr);

// part: K-split partial logits, router_splits(T, E, D) x T x E fp32 (unused
// and may be null when that is 1).
int router_splits(int T, int E, int D);
int launch_router(int T, int E, int D, int ng, int tg, int K, float route_scale,
                  const uint16_t* X, const float* Wr, const float* bcorr, float* logits,
                  int32_t* idx, float* w, float* part, unsigned* ctr, hipStream_t st);
bool boundary_router_fused(int T, int E, int D);
int launch_boundary_router(int T, int D, const uint16_t* y, const uint16_t* w_post, uint16_t* h,
                           const uint16_t* w_pre, uint16_t* x_out, int n, float eps, int E,
                           int ng, int tg, int K, float route_scale, const float* Wr,
                           const float* bcorr, float* logits, int32_t* idx, float* w,
                           float* part, unsigned* ctr, hipStream_t st);

// many-token (prefill) path
constexpr int kGemvMaxT = 4;  // T above this runs on the matrix-core kernels
// Attention calls of at most this many tokens, averaging at most 4 per cache
// slot (a batch of decode steps), run split-K per token like single-token
// decode; longer calls (prefill chunks) run the flash kernel.
constexpr int kDecodeBatchMaxT = 256;
int gemm_grouped_rows(int M, int E);  // tile rows of the grouped expert GEMMs
// part: fp32 split-K partials of gemm_split_bytes(M, N, K) bytes for short,
// wide products (nullptr: no split)
size_t gemm_split_bytes(int M, int N, int K);
int launch_gemm_bf16(int M, int N, int K, const uint16_t* A, int lda, const uint16_t* B, int ldb,
                     uint16_t* out, int ldo, uint16_t* out2, int ldo2, int n1, float* part,
                     hipStream_t st);
int launch_gemm_swiglu(int M, int F, int K, const uint16_t* A, int lda, const int32_t* gather,
                       const uint16_t* B, const int32_t* seg_off, const int32_t* tile_off, int E,
                       long long b_stride, int max_mtiles, uint16_t* act, float* part,
                       hipStream_t st, const uint16_t* B_last = nullptr);
// B_last (grouped mode): the weights of segment E - 1 in place of
// B + (E - 1) * b_stride (the shared expert after the routed ones)
int launch_gemm_f32(int M, int N, int K, const uint16_t* A, int lda, const uint16_t* B,
                    const int32_t* seg_off, const int32_t* tile_off, int E, long long b_stride,
                    int max_mtiles, float* out, int ldo, hipStream_t st,
                    const uint16_t* B_last = nullptr);
// Routing permutation over T * spt (token, slot) pairs: slots 0..K-1 the routed
// experts of idx, slot K (spt = K + 1) the shared expert as segment E.
// counts: moe_route_chunks(T * spt) x (E + 1) int32 of scratch; seg_off and
// tile_off: E + 2 entries.
int moe_route_chunks(int P);
int launch_moe_route(int T, int K, int spt, int E, const int32_t* idx, int tile_rows,
                     int32_t* counts, int32_t* seg_off, int32_t* tile_off, int32_t* perm,
                     int32_t* inv, hipStream_t st);
int launch_moe_combine(int T, int K, int spt, int E, int D, const float* out, const int32_t* inv,
                       const float* w, const int32_t* idx, uint16_t* y, hipStream_t st);
int launch_gate(int T, int Hq, int hd, const uint16_t* o, const uint16_t* g, const uint16_t* b,
                uint16_t* z, hipStream_t st);
// the many-token attention kernel covers these GQA group / head-dim shapes
inline bool attn_prefill_ok(int grp, int hd) {
  int ntb = (grp <= 6) ? 2 : 1;
  while (256 * grp * ntb < 16 * hd) ++ntb;
  return grp >= 1 && grp * ntb <= 12;
}
int launch_attn_prefill(int T, int Hq, int Hkv, int hd, int swa, int window, int fp8,
                        const uint16_t* q, const int32_t* pos, const int32_t* seq,
                        const void* kc, const void* vc, float k_scale, float v_scale, int S,
                        int Lmax, int npos, const float* sink, uint16_t* o, hipStream_t st);

int launch_hbm_read(const void* p, size_t bytes, unsigned* sink, hipStream_t st);

// device-side check flags (read and cleared by beam_check)
int gemv_read_clear_err();
int qk_read_clear_err();
int attn_read_clear_err();
int attnp_read_clear_err();
int moe_read_clear_err();
int mx_read_clear_err();

}  // namespace beam
