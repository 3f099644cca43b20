// FP32 router and DeepSeek-V3 grouped top-k ("Reflection Beam 1.0 on vLLM",
// MoE and residual stream section: sigmoid scores plus a correction bias pick
// the best 4 of 8 expert groups, then the top 8 experts; renormalised weights
// times 2.5; weights, accumulation and logits all FP32; optimisation change 4
// gives the router its own small-batch FP32 GEMM).
//
//  router_logits_gemv   few tokens: one workgroup per expert row, the fp32 row
//                       streamed once, K split over 4 waves, fixed-order sum
//  router_logits_gemm   many tokens: 64x64 fp32 tiles staged through LDS
//  router_topk          one workgroup per token, one thread per expert: group
//                       scores (sum of the two best biased scores), top groups
//                       by rank, top experts by block-wide arg-max rounds
//                       (ties to the lower index)
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

constexpr int EMAX = 1024;

// One workgroup per token, one thread per expert. Groups are chosen by rank
// (the number of groups that beat a group: larger score, or equal score and
// lower index); experts by topk rounds of a block-wide arg-max. Both break
// ties towards the lower index, and experts come out in selection order.
__global__ __launch_bounds__(EMAX) void router_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bcorr, int T, int E, int ng,
    int tg, int K, float route_scale, int32_t* __restrict__ idx, float* __restrict__ wout) {
  __shared__ float s_b[EMAX];
  __shared__ float g1[64], g2[64], gsc[64], ssel[32];
  __shared__ float wv_best[EMAX / 64];
  __shared__ int wi_best[EMAX / 64];
  const int t = blockIdx.x, e = threadIdx.x;
  const bool act = e < E;
  const int gs = E / ng;
  const int grp = act ? e / gs : 0;
  float sv = 0.f, sb = -INFINITY;
  if (act) {
    const float lg = logits[(size_t)t * E + e];
    sv = 1.0f / (1.0f + expf(-lg));
    sb = sv + (bcorr ? bcorr[e] : 0.f);
    s_b[e] = sb;
  }
  __syncthreads();
  // rank inside the group -> the group's two best biased scores
  if (act) {
    int r = 0;
    const int g0 = grp * gs;
    for (int m = g0; m < g0 + gs; ++m) {
      const float v = s_b[m];
      r += (v > sb) || (v == sb && m < e);
    }
    if (r == 0) g1[grp] = sb;
    if (r == 1) g2[grp] = sb;
  }
  __syncthreads();
  if (e < ng) gsc[e] = (gs >= 2) ? g1[e] + g2[e] : g1[e];
  __syncthreads();
  // group rank -> kept groups; candidates are the kept groups' experts
  bool kept = false;
  if (act) {
    const float my = gsc[grp];
    int r = 0;
    for (int h = 0; h < ng; ++h) r += (gsc[h] > my) || (gsc[h] == my && h < grp);
    kept = r < tg;
  }
  // topk rounds of a block-wide arg-max over the kept experts' biased scores
  float v = kept ? sb : -INFINITY;
  const int lane = e & 63, wave = e >> 6, nw = blockDim.x >> 6;
  for (int k = 0; k < K; ++k) {
    float bv = v;
    int bi = act ? e : 0x7fffffff;
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) {
      const float v2 = __shfl_xor(bv, o2, 64);
      const int i2 = __shfl_xor(bi, o2, 64);
      if (v2 > bv || (v2 == bv && i2 < bi)) {
        bv = v2;
        bi = i2;
      }
    }
    if (lane == 0) {
      wv_best[wave] = bv;
      wi_best[wave] = bi;
    }
    __syncthreads();
    float gv = wv_best[0];
    int gi = wi_best[0];
    for (int w2 = 1; w2 < nw; ++w2)
      if (wv_best[w2] > gv || (wv_best[w2] == gv && wi_best[w2] < gi)) {
        gv = wv_best[w2];
        gi = wi_best[w2];
      }
    if (e == gi) {
      v = -INFINITY;
      idx[(size_t)t * K + k] = e;
      ssel[k] = sv;
    }
    __syncthreads();
  }
  if (e < K) {
    float sum = 0.f;
    for (int k = 0; k < K; ++k) sum += ssel[k];
    wout[(size_t)t * K + e] = route_scale * ssel[e] / sum;
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
  const int threads = ((E + 63) / 64) * 64;
  hipLaunchKernelGGL(router_topk_kernel, dim3(T), dim3(threads), 0, st, logits, bcorr, T, E, ng,
                     tg, K, route_scale, idx, w);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace beam
