// Per-head Q/K RMSNorm with RoPE (sliding-window layers) or the SSMax query
// scale (NoPE layers), and the KV-cache write, in one kernel ("Reflection
// Beam 1.0 on vLLM": Attention section for the maths; optimisation changes 2
// and 6 for the fusion).
//
// One wave per head (qk_head). Input is the bf16 q|k|v projection.
#include "common.h"
#include "internal.h"
#include "qk_head.h"

namespace beam {

BEAM_ERR_FLAG_DECL(qk)
BEAM_ERR_FLAG_READER(qk)

// Tokens t0 + k * tstride for k < tpt (blockIdx.y = t0): the many-token path
// runs several tokens per wave and leaves the value heads to v_write_kernel
// (nh = Hq + Hkv); the few-token path has one token per wave and all heads.
__global__ __launch_bounds__(256) void qk_norm_pos_kvwrite_kernel(
    const uint16_t* __restrict__ qkv, int Hq, int Hkv, int hd,
    const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ seq, int mode,
    const float* __restrict__ rope_cs, uint16_t* __restrict__ q_out, void* __restrict__ kc,
    void* __restrict__ vc, int fp8, float ks, float vs, int S, int Lmax, float eps, int T,
    int nh, int tpt, int tstride) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int head = blockIdx.x * 4 + wave;
  const int nheads = Hq + 2 * Hkv;
  if (head >= nh) return;
  for (int k = 0; k < tpt; ++k) {
  const int t = blockIdx.y + k * tstride;
  if (t >= T) return;
  const int p = pos[t], s = seq[t];
  const bool slot_ok = (p >= 0 && p < Lmax && s >= 0 && s < S);
  if (!slot_ok && head == 0 && lane == 0)
    BEAM_RAISE(qk, (p < 0 || p >= Lmax) ? ERR_POS : ERR_SEQ);
  qk_head(qkv + (size_t)t * nheads * hd + (size_t)head * hd, head, Hq, Hkv, hd, wq, wk, p, s,
          slot_ok, mode, rope_cs, q_out + (size_t)t * Hq * hd, kc, vc, fp8, ks, vs, Lmax, eps);
  }
}

// Value heads of many tokens: one wave per (value head, 64 consecutive token
// indices), lane = token. Each lane reads its token's head row; then for every
// dim the 64 lanes store to V^T[seq][head][dim][pos], one run of consecutive
// positions when the tokens are consecutive positions of one sequence (a
// prefill chunk), so the stores coalesce.
__global__ __launch_bounds__(64) void v_write_kernel(const uint16_t* __restrict__ qkv, int Hq,
                                                     int Hkv, int hd,
                                                     const int32_t* __restrict__ pos,
                                                     const int32_t* __restrict__ seq,
                                                     void* __restrict__ vc, int fp8, float vs,
                                                     int S, int Lmax, int T) {
  const int j = blockIdx.x;
  const int t = blockIdx.y * 64 + threadIdx.x;
  if (t >= T) return;
  const int p = pos[t], s = seq[t];
  if (p < 0 || p >= Lmax || s < 0 || s >= S) return;  // flagged by the q/k kernel
  const int nheads = Hq + 2 * Hkv;
  const uint16_t* src = qkv + (size_t)t * nheads * hd + (size_t)(Hq + Hkv + j) * hd;
  const size_t col = (((size_t)s * Hkv + j) * hd) * (size_t)Lmax + p;  // V^T[s][j][0][p]
  for (int d0 = 0; d0 < hd; d0 += 8) {
    const uint4 u = ld16(src + d0);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t b = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      const size_t at = col + (size_t)(d0 + e) * Lmax;
      if (fp8) ((uint8_t*)vc)[at] = f2e4m3(__fdiv_rn(bf2f(b), vs));
      else ((uint16_t*)vc)[at] = b;
    }
  }
}

int launch_qk_epilogue(int T, int Hq, int Hkv, int hd, const uint16_t* qkv, const uint16_t* wq,
                       const uint16_t* wk, const int32_t* pos, const int32_t* seq, int mode,
                       const float* rope_cs, uint16_t* q_out, void* kc, void* vc, int fp8,
                       float k_scale, float v_scale, int S, int Lmax, float eps,
                       hipStream_t st) {
  if (T <= kGemvMaxT || (T <= kDecodeBatchMaxT && T <= 4 * S)) {
    // few tokens, or a batch of decode steps spread over many sequences: one
    // wave per (token, head), the value columns written by that wave
    const dim3 grid((Hq + 2 * Hkv + 3) / 4, T);
    hipLaunchKernelGGL(qk_norm_pos_kvwrite_kernel, grid, dim3(256), 0, st, qkv, Hq, Hkv, hd, wq,
                       wk, pos, seq, mode, rope_cs, q_out, kc, vc, fp8, k_scale, v_scale, S,
                       Lmax, eps, T, Hq + 2 * Hkv, 1, T);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  constexpr int TPT = 8;  // tokens per wave
  const int tb = (T + TPT - 1) / TPT;
  const dim3 grid((Hq + Hkv + 3) / 4, tb);
  hipLaunchKernelGGL(qk_norm_pos_kvwrite_kernel, grid, dim3(256), 0, st, qkv, Hq, Hkv, hd, wq,
                     wk, pos, seq, mode, rope_cs, q_out, kc, vc, fp8, k_scale, v_scale, S, Lmax,
                     eps, T, Hq + Hkv, TPT, tb);
  if (hipGetLastError() != hipSuccess) return -1;
  hipLaunchKernelGGL(v_write_kernel, dim3(Hkv, (T + 63) / 64), dim3(64), 0, st, qkv, Hq, Hkv,
                     hd, pos, seq, vc, fp8, v_scale, S, Lmax, T);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace beam
