// Sublayer boundary: post-norm -> depth-scaled residual add -> next pre-norm,
// one kernel per boundary ("Reflection Beam 1.0 on vLLM", MoE and residual
// stream section for the maths; optimisation change 1 for the fusion).
//
// One workgroup per token row. The row is held in registers between the two
// RMS reductions: 256 threads x up to 4 chunks of 8 bf16 covers D <= 8192.
// All statistics are fp32; every stored tensor is bf16.
#include "common.h"
#include "internal.h"

namespace beam {

constexpr int BT = 256;
constexpr int CPT = 4;  // 16-byte chunks per thread (D <= BT * CPT * 8)

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ void unpack8(uint4 u, float* f) {
  f[0] = bf_lo(u.x); f[1] = bf_hi(u.x); f[2] = bf_lo(u.y); f[3] = bf_hi(u.y);
  f[4] = bf_lo(u.z); f[5] = bf_hi(u.z); f[6] = bf_lo(u.w); f[7] = bf_hi(u.w);
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  return uint4{pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]), pack_bf2(f[4], f[5]),
               pack_bf2(f[6], f[7])};
}

// mode: 0 = entry (pre-norm of h only), 1 = post-norm + add, 2 = add without post-norm.
// Every input row is requested up front so the kernel pays one memory latency.
__global__ __launch_bounds__(BT) void boundary_kernel(
    int D, const uint16_t* __restrict__ y, const uint16_t* __restrict__ w_post,
    uint16_t* __restrict__ h, const uint16_t* __restrict__ w_pre,
    uint16_t* __restrict__ x_out, int mode, float c_h, float c_a, float eps) {
  __shared__ float red[4];
  const int nc = D >> 3;
  const size_t row = (size_t)blockIdx.x * D;
  uint4 yr[CPT], hr[CPT], wpr[CPT], wnr[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * BT;
    const bool in = c < nc;
    const uint4 z = {0u, 0u, 0u, 0u};
    hr[i] = in ? ld16(h + row + c * 8) : z;
    wnr[i] = in ? ld16(w_pre + c * 8) : z;
    yr[i] = (in && mode != 0) ? ld16(y + row + c * 8) : z;
    wpr[i] = (in && mode == 1) ? ld16(w_post + c * 8) : z;
  }
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
    const int c = threadIdx.x + i * BT;
    if (c < nc) {
      float wv[8], xo[8];
      unpack8(wnr[i], wv);
#pragma unroll
      for (int e = 0; e < 8; ++e) xo[e] = hv[i][e] * r * wv[e];
      if (mode != 0) *reinterpret_cast<uint4*>(h + row + c * 8) = pack8(hv[i]);
      *reinterpret_cast<uint4*>(x_out + row + c * 8) = pack8(xo);
    }
  }
}

int launch_boundary(int T, int D, const uint16_t* y, const uint16_t* w_post, uint16_t* h,
                    const uint16_t* w_pre, uint16_t* x_out, int n, float eps,
                    hipStream_t st) {
  int mode;
  float c_h = 1.f, c_a = 1.f;
  if (y == nullptr) {
    mode = 0;
  } else {
    mode = (w_post != nullptr) ? 1 : 2;
    if (n > 0) {
      c_h = (float)sqrt((double)(n - 1) / (double)n);
      c_a = (float)(1.0 / sqrt((double)n));
    }
  }
  hipLaunchKernelGGL(boundary_kernel, dim3(T), dim3(BT), 0, st, D, y, w_post, h, w_pre,
                     x_out, mode, c_h, c_a, eps);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace beam
