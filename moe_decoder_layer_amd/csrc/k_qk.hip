// Per-head Q/K RMSNorm with RoPE (sliding-window layers) or the SSMax query
// scale (NoPE layers), and the KV-cache write, in one kernel ("Reflection
// Beam 1.0 on vLLM": Attention section for the maths; optimisation changes 2
// and 6 for the fusion).
//
// One wave per head (qk_head). Input is the bf16 q|k|v projection. Position p
// goes to cache slot p mod Lmax (the identity unless the cache is a ring of
// Lmax slots accepting positions up to npos > Lmax).
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
    void* __restrict__ vc, int fp8, float ks, float vs, int S, int Lmax, int npos, float eps,
    int T, int nh, int tpt, int tstride) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int head = blockIdx.x * 4 + wave;
  const int nheads = Hq + 2 * Hkv;
  if (head >= nh) return;
  for (int k = 0; k < tpt; ++k) {
  const int t = blockIdx.y + k * tstride;
  if (t >= T) return;
  const int p = pos[t], s = seq[t];
  const bool slot_ok = (p >= 0 && p < npos && s >= 0 && s < S);
  if (!slot_ok && head == 0 && lane == 0)
    BEAM_RAISE(qk, (p < 0 || p >= npos) ? ERR_POS : ERR_SEQ);
  const int ps = slot_ok ? p % Lmax : 0;
  qk_head(qkv + (size_t)t * nheads * hd + (size_t)head * hd, head, Hq, Hkv, hd, wq, wk, p, ps,
          s, slot_ok, mode, rope_cs, q_out + (size_t)t * Hq * hd, kc, vc, fp8, ks, vs, Lmax,
          eps);
  }
}

// q and k heads of many tokens, head dim 128: sixteen lanes per (token, head),
// lane j holding elements 8j..8j+7 (one 16-byte load and store). The RMS
// statistic is a 16-lane reduction; lane j's rotate-half partner is lane j ^ 8.
// Slot u = token * (Hq + Hkv) + head.
__global__ __launch_bounds__(256) void qk_rows_kernel(
    const uint16_t* __restrict__ qkv, int Hq, int Hkv, const uint16_t* __restrict__ wq,
    const uint16_t* __restrict__ wk, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ seq, int mode, const float* __restrict__ rope_cs,
    uint16_t* __restrict__ q_out, void* __restrict__ kc, int fp8, float ks, int S, int Lmax,
    int npos, float eps, int T) {
  constexpr int HD = 128;
  const int lane = threadIdx.x & 63, j = lane & 15;
  const int nhq = Hq + Hkv, nheads = Hq + 2 * Hkv;
  const long long u = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  const bool live = u < (long long)T * nhq;
  const int t = live ? (int)(u / nhq) : 0, head = live ? (int)(u - (long long)t * nhq) : 0;
  const bool is_q = head < Hq;
  const int p = pos[t], s = seq[t];
  const bool slot_ok = (p >= 0 && p < npos && s >= 0 && s < S);
  if (live && !slot_ok && head == 0 && j == 0)
    BEAM_RAISE(qk, (p < 0 || p >= npos) ? ERR_POS : ERR_SEQ);
  // all loads first: the head's 8 values, the gains, this lane's cos/sin run
  const uint4 xv = ld16(qkv + (size_t)t * nheads * HD + (size_t)head * HD + 8 * j);
  const uint4 wv = ld16((is_q ? wq : wk) + 8 * j);
  const bool rot = (mode == 0) && slot_ok;
  float cs[8], sn[8];
  if (rot) {
    const float* row = rope_cs + (size_t)p * HD + 8 * (j & 7);
    const float4 c0 = *reinterpret_cast<const float4*>(row);
    const float4 c1 = *reinterpret_cast<const float4*>(row + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(row + HD / 2);
    const float4 s1 = *reinterpret_cast<const float4*>(row + HD / 2 + 4);
    cs[0] = c0.x; cs[1] = c0.y; cs[2] = c0.z; cs[3] = c0.w;
    cs[4] = c1.x; cs[5] = c1.y; cs[6] = c1.z; cs[7] = c1.w;
    sn[0] = s0.x; sn[1] = s0.y; sn[2] = s0.z; sn[3] = s0.w;
    sn[4] = s1.x; sn[5] = s1.y; sn[6] = s1.z; sn[7] = s1.w;
  }
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, ww[4] = {wv.x, wv.y, wv.z, wv.w};
  float x[8], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf_lo(xw[e]);
    x[2 * e + 1] = bf_hi(xw[e]);
    ss += x[2 * e] * x[2 * e] + x[2 * e + 1] * x[2 * e + 1];
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o, 64);
  const float r = rsqrtf(ss / HD + eps);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = x[2 * e] * r * bf_lo(ww[e]);
    x[2 * e + 1] = x[2 * e + 1] * r * bf_hi(ww[e]);
  }
  if (mode == 0) {  // RoPE at position p; every lane takes part in the exchange
    float pr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pr[e] = __shfl_xor(x[e], 8, 64);
    if (rot) {
      const bool first = j < 8;  // this lane holds a (elements < 64), the partner b
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[e] = first ? x[e] * cs[e] - pr[e] * sn[e] : x[e] * cs[e] + pr[e] * sn[e];
    }
  } else if (is_q) {  // SSMax: (1 + p/2048)^0.1 with the 1-based position p+1
    const float sc = __powf(1.0f + (float)(p + 1) * (1.0f / 2048.0f), 0.1f);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= sc;
  }
  if (!live) return;
  if (is_q) {
    uint4 o;
    o.x = pack_bf2(x[0], x[1]);
    o.y = pack_bf2(x[2], x[3]);
    o.z = pack_bf2(x[4], x[5]);
    o.w = pack_bf2(x[6], x[7]);
    *reinterpret_cast<uint4*>(q_out + ((size_t)t * Hq + head) * HD + 8 * j) = o;
    return;
  }
  if (!slot_ok) return;
  const size_t row =
      (((size_t)s * Hkv + (head - Hq)) * Lmax + p % Lmax) * HD + 8 * j;  // K[s][kv][slot]
  if (fp8) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= (uint32_t)f2e4m3(__fdiv_rn(x[e], ks)) << (8 * e);
      hi |= (uint32_t)f2e4m3(__fdiv_rn(x[4 + e], ks)) << (8 * e);
    }
    *reinterpret_cast<uint2*>((uint8_t*)kc + row) = uint2{lo, hi};
  } else {
    uint4 o;
    o.x = pack_bf2(x[0], x[1]);
    o.y = pack_bf2(x[2], x[3]);
    o.z = pack_bf2(x[4], x[5]);
    o.w = pack_bf2(x[6], x[7]);
    *reinterpret_cast<uint4*>((uint16_t*)kc + row) = o;
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
                                                     int S, int Lmax, int npos, int T) {
  const int j = blockIdx.x;
  const int t = blockIdx.y * 64 + threadIdx.x;
  if (t >= T) return;
  const int p = pos[t], s = seq[t];
  if (p < 0 || p >= npos || s < 0 || s >= S) return;  // flagged by the q/k kernel
  const int nheads = Hq + 2 * Hkv;
  const uint16_t* src = qkv + (size_t)t * nheads * hd + (size_t)(Hq + Hkv + j) * hd;
  const size_t col = (((size_t)s * Hkv + j) * hd) * (size_t)Lmax + p % Lmax;  // V^T[s][j][0][slot]
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
                       float k_scale, float v_scale, int S, int Lmax, int npos, float eps,
                       hipStream_t st) {
  if (T <= kGemvMaxT || (T <= kDecodeBatchMaxT && T <= 4 * S)) {
    // few tokens, or a batch of decode steps spread over many sequences: one
    // wave per (token, head), the value columns written by that wave
    const dim3 grid((Hq + 2 * Hkv + 3) / 4, T);
    hipLaunchKernelGGL(qk_norm_pos_kvwrite_kernel, grid, dim3(256), 0, st, qkv, Hq, Hkv, hd, wq,
                       wk, pos, seq, mode, rope_cs, q_out, kc, vc, fp8, k_scale, v_scale, S,
                       Lmax, npos, eps, T, Hq + 2 * Hkv, 1, T);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  if (hd == 128) {
    const long long items = (long long)T * (Hq + Hkv);  // (token, q or k head)
    hipLaunchKernelGGL(qk_rows_kernel, dim3((unsigned)((items + 15) / 16)), dim3(256), 0, st,
                       qkv, Hq, Hkv, wq, wk, pos, seq, mode, rope_cs, q_out, kc, fp8, k_scale,
                       S, Lmax, npos, eps, T);
  } else {
    constexpr int TPT = 8;  // tokens per wave
    const int tb = (T + TPT - 1) / TPT;
    const dim3 grid((Hq + Hkv + 3) / 4, tb);
    hipLaunchKernelGGL(qk_norm_pos_kvwrite_kernel, grid, dim3(256), 0, st, qkv, Hq, Hkv, hd, wq,
                       wk, pos, seq, mode, rope_cs, q_out, kc, vc, fp8, k_scale, v_scale, S,
                       Lmax, npos, eps, T, Hq + Hkv, TPT, tb);
  }
  if (hipGetLastError() != hipSuccess) return -1;
  hipLaunchKernelGGL(v_write_kernel, dim3(Hkv, (T + 63) / 64), dim3(64), 0, st, qkv, Hq, Hkv,
                     hd, pos, seq, vc, fp8, v_scale, S, Lmax, npos, T);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace beam
