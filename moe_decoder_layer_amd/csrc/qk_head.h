// One attention head of one token after the packed projection ("Reflection
// Beam 1.0 on vLLM", Attention section): per-head RMSNorm of q and k, RoPE
// (sliding-window layers) or the SSMax query scale (NoPE layers), and the
// cache write of k and v. Run by one full wave: lane i < d/2 holds elements i
// and i + d/2, one rotate-half pair, and the RMS statistic is one wave
// reduction.
#pragma once

#include "common.h"

namespace beam {

// The per-head RMSNorm of a q or k head (gain wq / wk over d), then RoPE at
// position p (mode 0, table row p: cos then sin) or, for q, the SSMax scale
// (1 + (p + 1) / 2048)^0.1 (mode 1). Lane i < d/2 gets elements i and
// i + d/2 in (a, b); other lanes get zeros. slot_ok false: no rotation.
__device__ __forceinline__ void qk_head_pair(const uint16_t* src, bool is_q, int hd,
                                             const uint16_t* __restrict__ wq,
                                             const uint16_t* __restrict__ wk, int p,
                                             bool slot_ok, int mode,
                                             const float* __restrict__ rope_cs, float eps,
                                             float& a, float& b) {
  const int lane = threadIdx.x & 63;
  const int half = hd >> 1;
  const bool act = lane < half;
  a = act ? bf2f(src[lane]) : 0.f;
  b = act ? bf2f(src[lane + half]) : 0.f;
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
}

// head in [0, Hq + 2 Hkv): q heads, then k heads, then v heads. src: the
// head's d bf16 projection values; q_row: the token's q output [Hq][d]; p the
// position (RoPE, SSMax), ps its cache slot (p mod Lmax).
__device__ __forceinline__ void qk_head(const uint16_t* src, int head, int Hq, int Hkv, int hd,
                                        const uint16_t* __restrict__ wq,
                                        const uint16_t* __restrict__ wk, int p, int ps, int s,
                                        bool slot_ok, int mode,
                                        const float* __restrict__ rope_cs, uint16_t* q_row,
                                        void* kc, void* vc, int fp8, float ks, float vs,
                                        int Lmax, float eps) {
  const int lane = threadIdx.x & 63;
  const int half = hd >> 1;
  const bool act = lane < half;
  float a = act ? bf2f(src[lane]) : 0.f;
  float b = act ? bf2f(src[lane + half]) : 0.f;
  if (head >= Hq + Hkv) {  // value head: stored as produced (bf16), or quantised
    if (!slot_ok || !act) return;
    const int j = head - Hq - Hkv;
    // V^T[s][j][dim][slot]
    const size_t col = ((size_t)s * Hkv + j) * (size_t)hd * (size_t)Lmax + (size_t)ps;
    if (fp8) {
      uint8_t* v = (uint8_t*)vc;
      v[col + (size_t)lane * Lmax] = f2e4m3(__fdiv_rn(a, vs));
      v[col + (size_t)(lane + half) * Lmax] = f2e4m3(__fdiv_rn(b, vs));
    } else {
      uint16_t* v = (uint16_t*)vc;
      v[col + (size_t)lane * Lmax] = src[lane];
      v[col + (size_t)(lane + half) * Lmax] = src[lane + half];
    }
    return;
  }
  const bool is_q = head < Hq;
  qk_head_pair(src, is_q, hd, wq, wk, p, slot_ok, mode, rope_cs, eps, a, b);
  if (is_q) {
    if (act) {
      uint16_t* qo = q_row + (size_t)head * hd;
      qo[lane] = f2bf(a);
      qo[lane + half] = f2bf(b);
    }
    return;
  }
  if (!slot_ok || !act) return;
  const int j = head - Hq;
  const size_t row = (((size_t)s * Hkv + j) * Lmax + ps) * hd;  // K[s][j][slot][:]
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

}  // namespace beam
