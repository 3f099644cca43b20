// Per-head Q/K RMSNorm with RoPE (sliding-window layers) or the SSMax query
// scale (NoPE layers), and the KV-cache write, in one kernel ("Reflection
// Beam 1.0 on vLLM": Attention section for the maths; optimisation changes 2
// and 6 for the fusion).
//
// One wave per head: lane i < d/2 holds elements i and i + d/2, which are
// exactly one rotate-half pair, so RoPE needs no lane exchange. The head's
// RMS statistic is one wave reduction. Input is the bf16 q|k|v projection.
#include "common.h"
#include "internal.h"

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
  const int half = hd >> 1;
  const bool act = lane < half;
  const int p = pos[t], s = seq[t];
  const bool slot_ok = (p >= 0 && p < Lmax && s >= 0 && s < S);
  if (!slot_ok && head == 0 && lane == 0)
    BEAM_RAISE(qk, (p < 0 || p >= Lmax) ? ERR_POS : ERR_SEQ);

  const uint16_t* src = qkv + (size_t)t * nheads * hd + (size_t)head * hd;
  float a = act ? bf2f(src[lane]) : 0.f;
  float b = act ? bf2f(src[lane + half]) : 0.f;

  if (head >= Hq + Hkv) {  // value head: stored as produced (bf16), or quantised
    if (!slot_ok || !act) continue;
    const int j = head - Hq - Hkv;
    const size_t col = (((size_t)s * Hkv + j) * hd) * (size_t)Lmax + p;  // V^T[s][j][dim][p]
    if (fp8) {
      uint8_t* v = (uint8_t*)vc;
      v[col + (size_t)lane * Lmax] = f2e4m3(__fdiv_rn(a, vs));
      v[col + (size_t)(lane + half) * Lmax] = f2e4m3(__fdiv_rn(b, vs));
    } else {
      uint16_t* v = (uint16_t*)vc;
      v[col + (size_t)lane * Lmax] = src[lane];
      v[col + (size_t)(lane + half) * Lmax] = src[lane + half];
    }
    continue;
  }
  const bool is_q = head < Hq;
  // gains and the RoPE row are requested before the reduction needs `a`, `b`
  const uint16_t* w = is_q ? wq : wk;
  const float wa = act ? bf2f(w[lane]) : 0.f, wb = act ? bf2f(w[lane + half]) : 0.f;
  const bool rot = (mode == 0) && slot_ok && act;
  const float c = rot ? rope_cs[(size_t)p * hd + lane] : 1.f;
  const float sn = rot ? rope_cs[(size_t)p * hd + half + lane] : 0.f;
  const float r = rsqrtf(wave_sum(a * a + b * b) / hd + eps);
  if (act) {
    a = a * r * wa;
    b = b * r * wb;
    if (mode == 0) {  // RoPE at position p (table row p: cos then sin)
      if (slot_ok) {
        const float a2 = a * c - b * sn;
        const float b2 = b * c + a * sn;
        a = a2;
        b = b2;
      }
    } else if (is_q) {  // SSMax: (1 + p/2048)^0.1 with the 1-based position p+1
      const float sc = __powf(1.0f + (float)(p + 1) * (1.0f / 2048.0f), 0.1f);
      a *= sc;
      b *= sc;
    }
  }
  if (is_q) {
    if (act) {
      uint16_t* qo = q_out + ((size_t)t * Hq + head) * hd;
      qo[lane] = f2bf(a);
      qo[lane + half] = f2bf(b);
    }
    continue;
  }
  if (!slot_ok || !act) continue;
  const int j = head - Hq;
  const size_t row = (((size_t)s * Hkv + j) * Lmax + p) * hd;  // K[s][j][p][:]
  if (fp8) {
    uint8_t* k = (uint8_t*)kc;
    k[row + lane] = f2e4m3(__fdiv_rn(a, ks));
    k[row + lane + half] = f2e4m3(__fdiv_rn(b, ks));
  } else {
    uint16_t* k = (uint16_t*)kc;
    k[row + lane] = f2bf(a);
    k[row + lane + half] = f2bf(b);
  }
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
  if (T <= kGemvMaxT) {
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
