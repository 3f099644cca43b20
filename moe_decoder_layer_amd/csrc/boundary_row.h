// One sublayer boundary row in registers ("Reflection Beam 1.0 on vLLM", MoE
// and residual stream section): post-norm of the sublayer output, the
// depth-scaled residual add, and the next pre-norm, for a workgroup of BT
// threads, each holding CPT chunks of 8 bf16 (D <= BT * CPT * 8). Shared by the
// boundary kernel and by kernels that run a boundary as their prologue, so
// every path rounds identically.
#pragma once

#include "common.h"

namespace beam {

template <int BT, int CPT>
struct BoundaryRow {
  uint4 yr[CPT], hr[CPT], wpr[CPT], wnr[CPT];

  // mode: 0 = entry (pre-norm of h only), 1 = post-norm + add, 2 = add
  // without post-norm. Every input chunk is requested before any is used.
  __device__ __forceinline__ void load(int D, const uint16_t* __restrict__ y,
                                       const uint16_t* __restrict__ w_post,
                                       const uint16_t* __restrict__ h,
                                       const uint16_t* __restrict__ w_pre, int mode) {
    const int nc = D >> 3;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * BT;
      const bool in = c < nc;
      const uint4 z = {0u, 0u, 0u, 0u};
      hr[i] = in ? ld16(h + c * 8) : z;
      wnr[i] = in ? ld16(w_pre + c * 8) : z;
      yr[i] = (in && mode != 0) ? ld16(y + c * 8) : z;
      wpr[i] = (in && mode == 1) ? ld16(w_post + c * 8) : z;
    }
  }

  static __device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float s = red[0];
#pragma unroll
    for (int k = 1; k < BT / 64; ++k) s += red[k];
    return s;
  }
  static __device__ __forceinline__ void unpack8(uint4 u, float* f) {
    f[0] = bf_lo(u.x); f[1] = bf_hi(u.x); f[2] = bf_lo(u.y); f[3] = bf_hi(u.y);
    f[4] = bf_lo(u.z); f[5] = bf_hi(u.z); f[6] = bf_lo(u.w); f[7] = bf_hi(u.w);
  }
  static __device__ __forceinline__ uint4 pack8(const float* f) {
    return uint4{pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]), pack_bf2(f[4], f[5]),
                 pack_bf2(f[6], f[7])};
  }

  // hn = the new residual row (bf16), xo = its pre-norm (bf16); red: >= BT/64
  // floats of LDS. Every thread of the workgroup must call this.
  __device__ __forceinline__ void compute(int D, int mode, float c_h, float c_a, float eps,
                                          float* red, uint4 (&hn)[CPT], uint4 (&xo)[CPT]) {
    const int nc = D >> 3;
    float hv[CPT][8];
    if (mode == 1) {
      float yv[CPT][8];
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        unpack8(yr[i], yv[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += yv[i][e] * yv[i][e];
      }
      const float r = rsqrtf(block_sum(ss, red) / D + eps);
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        float wv[8], hh[8];
        unpack8(wpr[i], wv);
        unpack8(hr[i], hh);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = round_bf(yv[i][e] * r * wv[e]);
          hv[i][e] = round_bf(c_h * hh[e] + c_a * a);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        unpack8(hr[i], hv[i]);
        if (mode == 2) {
          float yv[8];
          unpack8(yr[i], yv);
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[i][e] = round_bf(c_h * hv[i][e] + c_a * yv[e]);
        }
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * BT;
      if (c < nc) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += hv[i][e] * hv[i][e];
      }
    }
    const float r = rsqrtf(block_sum(ss, red) / D + eps);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      float wv[8], x8[8];
      unpack8(wnr[i], wv);
#pragma unroll
      for (int e = 0; e < 8; ++e) x8[e] = hv[i][e] * r * wv[e];
      hn[i] = pack8(hv[i]);
      xo[i] = pack8(x8);
    }
  }
};

// Residual coefficients of the n-th add: sqrt((n-1)/n) and 1/sqrt(n) (1, 1
// for n = 0, the plain add).
inline void boundary_coefs(int n, float* c_h, float* c_a) {
  *c_h = 1.f;
  *c_a = 1.f;
  if (n > 0) {
    *c_h = (float)sqrt((double)(n - 1) / (double)n);
    *c_a = (float)(1.0 / sqrt((double)n));
  }
}

}  // namespace beam
