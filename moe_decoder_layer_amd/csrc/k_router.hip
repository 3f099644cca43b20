// FP32 router and DeepSeek-V3 grouped top-k ("Reflection Beam 1.0 on vLLM",
// MoE and residual stream section: sigmoid scores plus a correction bias pick
// the best 4 of 8 expert groups, then the top 8 experts; renormalised weights
// times 2.5; weights, accumulation and logits all FP32; optimisation change 4
// gives the router its own small-batch FP32 GEMM).
//
//  router_logits_gemv   few tokens: one workgroup per expert row, the fp32 row
//                       streamed once, K split over 4 waves, fixed-order sum
//  router_logits_gemm   many tokens: 64x64 fp32 tiles staged through LDS
//  router_topk          one wave per token: group scores (sum of the two best
//                       biased scores), top groups, top experts by wave-wide
//                       arg-max with ties to the lower index
#include "common.h"
#include "internal.h"

namespace beam {

constexpr int RT = 256;

template <int TT>
__global__ __launch_bounds__(RT) void router_logits_gemv_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ Wr, int T, int E, int D,
    float* __restrict__ logits) {
  __shared__ float red[4][TT];
  const int e = blockIdx.x, t0 = blockIdx.y * TT;
  const float* w = Wr + (size_t)e * D;
  float acc[TT] = {};
  const int nc = D >> 2;  // float4 chunks
  for (int c = threadIdx.x; c < nc; c += RT) {
    const f32x4 wv = ld16f_nt(w + (size_t)c * 4);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t0 + t < T) {
        const uint2 xv = *reinterpret_cast<const uint2*>(X + (size_t)(t0 + t) * D + c * 4);
        float a = acc[t];
        a = __builtin_fmaf(bf_lo(xv.x), wv[0], a);
        a = __builtin_fmaf(bf_hi(xv.x), wv[1], a);
        a = __builtin_fmaf(bf_lo(xv.y), wv[2], a);
        a = __builtin_fmaf(bf_hi(xv.y), wv[3], a);
        acc[t] = a;
      }
    }
  }
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float v = wave_sum(acc[t]);
    if ((threadIdx.x & 63) == 0) red[wave][t] = v;
  }
  __syncthreads();
  if (threadIdx.x < TT && t0 + (int)threadIdx.x < T) {
    const int t = threadIdx.x;
    logits[(size_t)(t0 + t) * E + e] = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
  }
}

// 64 tokens x 64 experts per workgroup, k-steps of 16; each thread 4x4 outputs.
__global__ __launch_bounds__(RT) void router_logits_gemm_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ Wr, int T, int E, int D,
    float* __restrict__ logits) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tm = blockIdx.x * 64, en = blockIdx.y * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < D; k0 += 16) {
    for (int i = threadIdx.x; i < 64 * 16; i += RT) {
      const int r = i >> 4, k = i & 15;
      const int tt = tm + r, ee = en + r;
      const bool kin = k0 + k < D;
      As[k][r] = (tt < T && kin) ? bf2f(X[(size_t)tt * D + k0 + k]) : 0.f;
      Bs[k][r] = (ee < E && kin) ? Wr[(size_t)ee * D + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[k][ty * 4 + i];
        b[i] = Bs[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = __builtin_fmaf(a[i], b[jj], acc[i][jj]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int tt = tm + ty * 4 + i, ee = en + tx * 4 + jj;
      if (tt < T && ee < E) logits[(size_t)tt * E + ee] = acc[i][jj];
    }
}

// Wave-wide arg-max: larger value wins, equal values go to the lower index.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(v, o, 64);
    const int i2 = __shfl_xor(i, o, 64);
    if (v2 > v || (v2 == v && i2 < i)) {
      v = v2;
      i = i2;
    }
  }
}

constexpr int EMAX = 1024;

__global__ __launch_bounds__(RT) void router_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bcorr, int T, int E, int ng,
    int tg, int K, float route_scale, int32_t* __restrict__ idx, float* __restrict__ wout) {
  __shared__ float s_raw[4][EMAX];
  __shared__ float s_b[4][EMAX];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t < T) {
    for (int e = lane; e < E; e += 64) {
      const float lg = logits[(size_t)t * E + e];
      const float sv = 1.0f / (1.0f + expf(-lg));
      s_raw[wave][e] = sv;
      s_b[wave][e] = sv + (bcorr ? bcorr[e] : 0.f);
    }
  }
  __syncthreads();
  if (t >= T) return;
  const int gs = E / ng;
  // group score: the two largest biased scores of the group, summed
  float gsc = -INFINITY;
  if (lane < ng) {
    float b1 = -INFINITY, b2 = -INFINITY;
    for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
      const float v = s_b[wave][e];
      if (v > b1) {
        b2 = b1;
        b1 = v;
      } else if (v > b2) {
        b2 = v;
      }
    }
    gsc = (gs >= 2) ? b1 + b2 : b1;
  }
  uint64_t kept = 0;
  for (int r = 0; r < tg; ++r) {
    float v = gsc;
    int i = (lane < ng) ? lane : 1 << 30;
    wave_argmax(v, i);
    kept |= 1ull << i;
    if (lane == i) gsc = -INFINITY;
  }
  // candidates: experts of the kept groups; lane holds e = lane + 64*k
  constexpr int PER = EMAX / 64;
  float cand[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = lane + 64 * k;
    cand[k] = (e < E && ((kept >> (e / gs)) & 1ull)) ? s_b[wave][e] : -INFINITY;
  }
  int myidx = 0;
  float mys = 0.f;
  float ssum = 0.f;
  for (int r = 0; r < K; ++r) {
    float v = -INFINITY;
    int i = 1 << 30;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = lane + 64 * k;
      if (cand[k] > v || (cand[k] == v && e < i)) {
        v = cand[k];
        i = e;
      }
    }
    wave_argmax(v, i);
    if ((i & 63) == lane) {
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if (lane + 64 * k == i) cand[k] = -INFINITY;
    }
    const float si = s_raw[wave][i];
    ssum += si;
    if (lane == r) {
      myidx = i;
      mys = si;
    }
  }
  if (lane < K) {
    idx[(size_t)t * K + lane] = myidx;
    wout[(size_t)t * K + lane] = route_scale * mys / ssum;
  }
}

int launch_router(int T, int E, int D, int ng, int tg, int K, float route_scale,
                  const uint16_t* X, const float* Wr, const float* bcorr, float* logits,
                  int32_t* idx, float* w, hipStream_t st) {
  if (T <= 4) {
    hipLaunchKernelGGL((router_logits_gemv_kernel<4>), dim3(E, 1), dim3(RT), 0, st, X, Wr, T, E,
                       D, logits);
  } else {
    hipLaunchKernelGGL(router_logits_gemm_kernel, dim3((T + 63) / 64, (E + 63) / 64), dim3(RT),
                       0, st, X, Wr, T, E, D, logits);
  }
  if (hipGetLastError() != hipSuccess) return -1;
  hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), dim3(RT), 0, st, logits, bcorr, T, E,
                     ng, tg, K, route_scale, idx, w);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace beam
