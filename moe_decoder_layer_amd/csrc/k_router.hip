// FP32 router and DeepSeek-V3 grouped top-k ("Reflection Beam 1.0 on vLLM",
// MoE and residual stream section: sigmoid scores plus a correction bias pick
// the best 4 of 8 expert groups, then the top 8 experts; renormalised weights
// times 2.5; weights, accumulation and logits all FP32; optimisation change 4
// gives the router its own small-batch FP32 GEMM).
//
//  router_decode        few tokens: one wave per expert row, the fp32 row
//                       streamed once; the workgroup that finishes last runs
//                       the selection for every token (no second launch)
//  router_logits_gemm   many tokens: 64x64 fp32 tiles staged through LDS
//  router_topk          many tokens: one workgroup per token
// Selection (route_token), one thread per expert: group scores (sum of the two
// best biased scores), the top groups by rank, then the top experts by rank
// among the kept groups' best experts. A rank counts the candidates that beat
// a candidate (larger value, or equal value and lower index), so ties go to
// the lower index and the experts come out in descending biased-score order.
#include "boundary_row.h"
#include "common.h"
#include "internal.h"

namespace beam {

constexpr int RT = 256;

// 64 tokens x 64 experts per workgroup, each thread 4 x 4 outputs; K in
// blocks of 32 staged through LDS as fp32, the next block's 16-byte loads in
// flight while the current one is multiplied out. blockIdx.z = split of the
// K range (kc values each): split z writes its partial sums to
// logits + z * T * E (summed in split order by the selection kernel).
__global__ __launch_bounds__(RT) void router_logits_gemm_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ Wr, int T, int E, int D, int kc,
    float* __restrict__ logits) {
  constexpr int KB = 32;
  __shared__ float As[KB][64 + 4];
  __shared__ float Bs[KB][64 + 4];
  const int tm = blockIdx.x * 64, en = blockIdx.y * 64;
  const int kbeg = blockIdx.z * kc, kend = min(D, kbeg + kc);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  // loader roles: A row ra (token), 8 k from ka; B row rb (expert), 2 x 4 k from kb
  const int ra = threadIdx.x >> 2, ka = (threadIdx.x & 3) * 8;
  const int rb = threadIdx.x >> 2, kb = (threadIdx.x & 3) * 8;
  const bool aok = tm + ra < T, bok = en + rb < E;
  const uint16_t* ap = X + (size_t)min(tm + ra, T - 1) * D;
  const float* bp = Wr + (size_t)min(en + rb, E - 1) * D;
  // D % 8 == 0; a block past kend reads zeros (k beyond D is clamped, masked)
  auto load = [&](int k0, uint4& av, float4& b0, float4& b1) {
    const int k = k0 + ka, kk = k0 + kb;
    av = (aok && k < kend) ? ld16(ap + k) : uint4{0u, 0u, 0u, 0u};
    if (bok && kk < kend) {
      b0 = *reinterpret_cast<const float4*>(bp + kk);
      b1 = *reinterpret_cast<const float4*>(bp + kk + 4);
    } else {
      b0 = b1 = float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store = [&](const uint4& av, const float4& b0, const float4& b1) {
    const uint32_t w[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      As[ka + 2 * i][ra] = __uint_as_float(w[i] << 16);
      As[ka + 2 * i + 1][ra] = __uint_as_float(w[i] & 0xffff0000u);
    }
    Bs[kb + 0][rb] = b0.x; Bs[kb + 1][rb] = b0.y; Bs[kb + 2][rb] = b0.z; Bs[kb + 3][rb] = b0.w;
    Bs[kb + 4][rb] = b1.x; Bs[kb + 5][rb] = b1.y; Bs[kb + 6][rb] = b1.z; Bs[kb + 7][rb] = b1.w;
  };
  // Sums in three levels: each 32-term slab from zero, eight slabs into a
  // 256-term group, the groups into the total. A plain running sum over D
  // terms rounds at the magnitude of the whole partial sum on every add (an
  // error of order 2^-24 * |logit| * sqrt(D / 2)); this way only the D / 256
  // group adds do.
  float acc[4][4] = {}, grp[4][4] = {};
  int nslab = 0;
  uint4 av;
  float4 b0, b1;
  load(kbeg, av, b0, b1);
  for (int k0 = kbeg; k0 < kend; k0 += KB) {
    store(av, b0, b1);
    __syncthreads();
    if (k0 + KB < kend) load(k0 + KB, av, b0, b1);
    float sl[4][4] = {};
#pragma unroll 8
    for (int k = 0; k < KB; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[k][ty * 4 + i];
        b[i] = Bs[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sl[i][jj] = __builtin_fmaf(a[i], b[jj], sl[i][jj]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) grp[i][jj] += sl[i][jj];
    if (++nslab == 8) {
      nslab = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          acc[i][jj] += grp[i][jj];
          grp[i][jj] = 0.f;
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[i][jj] += grp[i][jj];
  float* out = logits + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int tt = tm + ty * 4 + i, ee = en + tx * 4 + jj;
      if (tt < T && ee < E) out[(size_t)tt * E + ee] = acc[i][jj];
    }
}

// Splits of the K range for the many-token logits GEMM: enough workgroups to
// cover the chip when there are few token tiles, each split a multiple of 32.
int router_splits(int T, int E, int D) {
  const int tiles = ((T + 63) / 64) * ((E + 63) / 64);
  int s = 1;
  while (s * 2 * tiles <= 256 && D % (s * 2 * 32) == 0 && D / (s * 2) >= 128) s *= 2;
  return s;
}

constexpr int EMAX = 1024;

// Number of the n keys k[0, n) in LDS above `mine`. For even n (k 16-byte
// aligned) they are read two to a 16-byte vector, up to 16 keys requested
// before the first comparison, so the reads overlap.
__device__ __forceinline__ int count_above(const uint64_t* k, int n, uint64_t mine) {
  int r = 0;
  if ((n & 1) == 0) {
    typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
    for (int j0 = 0; j0 < n; j0 += 16) {
      u64x2 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (j0 + 2 * q < n) v[q] = *reinterpret_cast<const u64x2*>(k + j0 + 2 * q);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (j0 + 2 * q < n) r += (int)(v[q][0] > mine) + (int)(v[q][1] > mine);
    }
  } else {
    for (int j = 0; j < n; ++j) r += (int)(k[j] > mine);
  }
  return r;
}

// Grouped top-k of one token, one thread per expert (E <= blockDim.x).
// lg: the token's logits; bias: this thread's correction bias (0 when none).
// Each expert's rank key is its biased score made order-preserving as an
// unsigned high word, over 0xFFFFFFFF - e in the low word: a key is above
// another exactly when its score is larger, or equal with a lower index (the
// rank rule), so every rank is a count of larger keys.
// LDS scratch (16-byte aligned): key, ckey >= E entries, g1, g2 >= ng,
// ssel >= K, red >= 32.
// An expert among the overall top K is among the top K of its own group, so
// the final ranking only runs over each kept group's best min(K, group size).
__device__ __forceinline__ void route_token(const float* lg, float bias, int E, int ng, int tg,
                                            int K, float route_scale, int32_t* idx_t, float* w_t,
                                            uint64_t* key, uint64_t* ckey, float* g1, float* g2,
                                            float* ssel, int* red) {
  const int e = threadIdx.x;
  const bool act = e < E;
  float sv = 0.f, sb = -INFINITY;
  uint64_t my = 0;  // below every expert's key
  if (act) {
    sv = 1.0f / (1.0f + expf(-lg[e]));
    sb = sv + bias;
    const uint32_t u = __float_as_uint(sb + 0.0f);  // -0 -> +0: equal scores, equal words
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    my = ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
  }
  if (ng == 1 || tg >= ng) {
    // Every group kept: the top K keys, in K rounds of a workgroup argmax;
    // a lane whose expert is taken drops its key to 0.
    uint64_t* red64 = reinterpret_cast<uint64_t*>(red);  // one key per wave (<= 16)
    const int nw = (blockDim.x + 63) >> 6, wave = threadIdx.x >> 6;
    for (int r = 0; r < K; ++r) {
      uint64_t b = my;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const uint64_t ob = __shfl_xor(b, o, 64);
        b = ob > b ? ob : b;
      }
      if ((threadIdx.x & 63) == 0) red64[wave] = b;
      __syncthreads();
      b = red64[0];
      for (int w = 1; w < nw; ++w) b = red64[w] > b ? red64[w] : b;
      __syncthreads();  // red is rewritten next round
      if (act && b == my) {
        idx_t[r] = e;
        ssel[r] = sv;
        my = 0;
      }
    }
    __syncthreads();
    if (e < K) {
      float sum = 0.f;
      for (int k = 0; k < K; ++k) sum += ssel[k];
      w_t[e] = route_scale * ssel[e] / sum;
    }
    __syncthreads();  // the LDS arrays are reused for the next token
    return;
  }
  const int gs = E / ng;
  const int kc = min(K, gs);  // candidates per kept group
  const int nc = tg * kc;     // <= E
  const int grp = act ? e / gs : 0;
  if (act) key[e] = my;
  if (e < nc) ckey[e] = 0;  // slots a group cannot fill stay empty (below every key)
  __syncthreads();
  // rank inside the group; the two best give the group's score
  int rin = 0;
  if (act) {
    rin = count_above(key + grp * gs, gs, my);
    if (rin == 0) g1[grp] = sb;
    if (rin == 1) g2[grp] = sb;
  }
  __syncthreads();
  bool cand = false;  // in a kept group and among its best kc
  if (act && rin < kc) {
    const float mine = (gs >= 2) ? g1[grp] + g2[grp] : g1[grp];
    int rg = 0;
    for (int h = 0; h < ng; ++h) {
      const float sc = (gs >= 2) ? g1[h] + g2[h] : g1[h];
      rg += (int)((sc > mine) | ((sc == mine) & (h < grp)));
    }
    cand = rg < tg;
    if (cand) ckey[rg * kc + rin] = my;
  }
  __syncthreads();
  // final rank among the candidates
  if (cand) {
    const int r = count_above(ckey, nc, my);
    if (r < K) {
      idx_t[r] = e;
      ssel[r] = sv;
    }
  }
  __syncthreads();
  if (e < K) {
    float sum = 0.f;
    for (int k = 0; k < K; ++k) sum += ssel[k];
    w_t[e] = route_scale * ssel[e] / sum;
  }
  __syncthreads();  // the LDS arrays are reused for the next token
}

// part != nullptr: the logits are the sum over nsplit partial arrays, added in
// split order and written to logits first.
__global__ __launch_bounds__(EMAX) void router_topk_kernel(
    float* __restrict__ logits, const float* __restrict__ part, int nsplit,
    const float* __restrict__ bcorr, int T, int E, int ng, int tg, int K, float route_scale,
    int32_t* __restrict__ idx, float* __restrict__ wout) {
  __shared__ __align__(16) uint64_t key[EMAX], ckey[EMAX];
  __shared__ __align__(16) float g1[64], g2[64], ssel[32];
  __shared__ __align__(16) int sred[32];
  const int t = blockIdx.x;
  if (part != nullptr && (int)threadIdx.x < E) {
    // eight partials requested at a time, added in split order
    float v = 0.f;
    for (int z0 = 0; z0 < nsplit; z0 += 8) {
      float pz[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pz[i] = z0 + i < nsplit ? part[((size_t)(z0 + i) * T + t) * E + threadIdx.x] : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (z0 + i < nsplit) v += pz[i];
    }
    logits[(size_t)t * E + threadIdx.x] = v;
  }
  const float bias = (bcorr && (int)threadIdx.x < E) ? bcorr[threadIdx.x] : 0.f;
  route_token(logits + (size_t)t * E, bias, E, ng, tg, K, route_scale, idx + (size_t)t * K,
              wout + (size_t)t * K, key, ckey, g1, g2, ssel, sred);
}

// Few tokens: wave w of workgroup b computes the logits of expert 4b + w for
// up to TT tokens, each lane requesting its MAXC float4 chunks of the row per
// pass before using any (addresses past the row are clamped and their values
// zeroed, so the loads carry no branches). The workgroup that finishes last
// runs the selection for every token (E <= RT).
template <int TT, int MAXC>
__global__ __launch_bounds__(RT) void router_decode_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ Wr, int T, int E, int D,
    float* logits, const float* __restrict__ bcorr, int ng, int tg, int K, float route_scale,
    int32_t* __restrict__ idx, float* __restrict__ wout, unsigned* ctr) {
  __shared__ __align__(16) uint64_t key[RT], ckey[RT];
  __shared__ __align__(16) float g1[64], g2[64], ssel[32];
  __shared__ __align__(16) int sred[32];
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // the selection needs the bias in whichever workgroup ends up last
  const float bias = (bcorr && (int)threadIdx.x < E) ? bcorr[threadIdx.x] : 0.f;
  const int e = blockIdx.x * 4 + wave;
  const float* w = Wr + (size_t)min(e, E - 1) * D;
  const int nc = D >> 2;  // float4 chunks of a row
  float acc[TT] = {};
  for (int c0 = 0; c0 < nc; c0 += MAXC * 64) {
    f32x4 wv[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = c0 + lane + 64 * i;
      wv[i] = ld16f_nt(w + (size_t)min(c, nc - 1) * 4);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t < T) {
        uint2 xv[MAXC];
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
          const int c = c0 + lane + 64 * i;
          xv[i] = *reinterpret_cast<const uint2*>(X + (size_t)t * D + min(c, nc - 1) * 4);
        }
        float a = acc[t];
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
          if (c0 + lane + 64 * i < nc) {
            a = __builtin_fmaf(bf_lo(xv[i].x), wv[i][0], a);
            a = __builtin_fmaf(bf_hi(xv[i].x), wv[i][1], a);
            a = __builtin_fmaf(bf_lo(xv[i].y), wv[i][2], a);
            a = __builtin_fmaf(bf_hi(xv[i].y), wv[i][3], a);
          }
        }
        acc[t] = a;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float v = wave_sum(acc[t]);
    if (lane == 0 && t < T && e < E) st_dev(logits + (size_t)t * E + e, v);
  }
  if (!last_arrival(ctr, gridDim.x, &s_last)) return;
  for (int t = 0; t < T; ++t)
    route_token(logits + (size_t)t * E, bias, E, ng, tg, K, route_scale, idx + (size_t)t * K,
                wout + (size_t)t * K, key, ckey, g1, g2, ssel, sred);
}

// One token: the attention-side sublayer boundary as the router's prologue.
// Each workgroup requests its expert rows first, computes the boundary row
// (new residual h and its pre-norm x) while they arrive, keeps x in LDS as the
// GEMV input, and the last workgroup to finish (after every workgroup has read
// the old h) stores h and x and runs the selection. Products and sums follow
// router_decode_kernel's order, so both paths give identical logits.
template <int MAXC>
__global__ __launch_bounds__(RT) void boundary_router_kernel(
    int D, const uint16_t* __restrict__ y, const uint16_t* __restrict__ w_post, uint16_t* h,
    const uint16_t* __restrict__ w_pre, uint16_t* __restrict__ x_out, int mode, float c_h,
    float c_a, float eps, const float* __restrict__ Wr, int E, float* logits,
    const float* __restrict__ bcorr, int ng, int tg, int K, float route_scale,
    int32_t* __restrict__ idx, float* __restrict__ wout, unsigned* ctr) {
  constexpr int CPT = 4;  // D <= RT * CPT * 8
  extern __shared__ __align__(16) uint16_t xs[];  // the token's pre-normed row
  __shared__ float red[RT / 64];
  __shared__ __align__(16) uint64_t key[RT], ckey[RT];
  __shared__ __align__(16) float g1[64], g2[64], ssel[32];
  __shared__ __align__(16) int sred[32];
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  const float* w = Wr + (size_t)min(e, E - 1) * D;
  const int nc = D >> 2;  // float4 chunks of a row (nc <= 64 * MAXC)
  f32x4 wv[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) wv[i] = ld16f_nt(w + (size_t)min(lane + 64 * i, nc - 1) * 4);
  const float bias = (bcorr && (int)threadIdx.x < E) ? bcorr[threadIdx.x] : 0.f;

  BoundaryRow<RT, CPT> br;
  br.load(D, y, w_post, h, w_pre, mode);
  uint4 hn[CPT], xo[CPT];
  br.compute(D, mode, c_h, c_a, eps, red, hn, xo);
  const int nc8 = D >> 3;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * RT;
    if (c < nc8) *reinterpret_cast<uint4*>(xs + c * 8) = xo[i];
  }
  __syncthreads();
  // every x chunk is read before the first product (chunks past the row read
  // the last one and are left out), so no branch waits on its own read
  uint2 xv[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i)
    xv[i] = *reinterpret_cast<const uint2*>(xs + min(lane + 64 * i, nc - 1) * 4);
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    if (lane + 64 * i < nc) {
      a = __builtin_fmaf(bf_lo(xv[i].x), wv[i][0], a);
      a = __builtin_fmaf(bf_hi(xv[i].x), wv[i][1], a);
      a = __builtin_fmaf(bf_lo(xv[i].y), wv[i][2], a);
      a = __builtin_fmaf(bf_hi(xv[i].y), wv[i][3], a);
    }
  }
  const float v = wave_sum(a);
  if (lane == 0 && e < E) st_dev(logits + e, v);
  if (!last_arrival(ctr, gridDim.x, &s_last)) return;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * RT;
    if (c < nc8) {
      if (mode != 0) *reinterpret_cast<uint4*>(h + c * 8) = hn[i];
      *reinterpret_cast<uint4*>(x_out + c * 8) = xo[i];
    }
  }
  route_token(logits, bias, E, ng, tg, K, route_scale, idx, wout, key, ckey, g1, g2, ssel, sred);
}

bool boundary_router_fused(int T, int E, int D) {
  return T == 1 && E <= RT && D % 8 == 0 && D <= 20 * 64 * 4 && D <= RT * 4 * 8;
}

int launch_boundary_router(int T, int D, const uint16_t* y, const uint16_t* w_post, uint16_t* h,
                           const uint16_t* w_pre, uint16_t* x_out, int n, float eps, int E,
                           int ng, int tg, int K, float route_scale, const float* Wr,
                           const float* bcorr, float* logits, int32_t* idx, float* w,
                           float* part, unsigned* ctr, hipStream_t st) {
  if (!boundary_router_fused(T, E, D)) {
    if (launch_boundary(T, D, y, w_post, h, w_pre, x_out, n, eps, st)) return -1;
    return launch_router(T, E, D, ng, tg, K, route_scale, x_out, Wr, bcorr, logits, idx, w, part,
                         ctr, st);
  }
  const int mode = (y == nullptr) ? 0 : (w_post != nullptr ? 1 : 2);
  float c_h, c_a;
  boundary_coefs(mode == 0 ? 0 : n, &c_h, &c_a);
  const dim3 grid((E + 3) / 4);
  const size_t sh = (size_t)D * 2;
  if (D <= 8 * 64 * 4)
    hipLaunchKernelGGL((boundary_router_kernel<8>), grid, dim3(RT), sh, st, D, y, w_post, h,
                       w_pre, x_out, mode, c_h, c_a, eps, Wr, E, logits, bcorr, ng, tg, K,
                       route_scale, idx, w, ctr);
  else
    hipLaunchKernelGGL((boundary_router_kernel<20>), grid, dim3(RT), sh, st, D, y, w_post, h,
                       w_pre, x_out, mode, c_h, c_a, eps, Wr, E, logits, bcorr, ng, tg, K,
                       route_scale, idx, w, ctr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_router(int T, int E, int D, int ng, int tg, int K, float route_scale,
                  const uint16_t* X, const float* Wr, const float* bcorr, float* logits,
                  int32_t* idx, float* w, float* part, unsigned* ctr, hipStream_t st) {
  if (T <= 4 && E <= RT) {
    const dim3 grid((E + 3) / 4);
    if (D <= 8 * 64 * 4)
      hipLaunchKernelGGL((router_decode_kernel<4, 8>), grid, dim3(RT), 0, st, X, Wr, T, E, D,
                         logits, bcorr, ng, tg, K, route_scale, idx, w, ctr);
    else
      hipLaunchKernelGGL((router_decode_kernel<4, 20>), grid, dim3(RT), 0, st, X, Wr, T, E, D,
                         logits, bcorr, ng, tg, K, route_scale, idx, w, ctr);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int ns = router_splits(T, E, D);
  if (ns > 1 && part == nullptr) return -1;
  const int kc = D / ns;
  hipLaunchKernelGGL(router_logits_gemm_kernel, dim3((T + 63) / 64, (E + 63) / 64, ns), dim3(RT),
                     0, st, X, Wr, T, E, D, kc, ns > 1 ? part : logits);
  if (hipGetLastError() != hipSuccess) return -1;
  const int threads = ((E + 63) / 64) * 64;
  hipLaunchKernelGGL(router_topk_kernel, dim3(T), dim3(threads), 0, st, logits,
                     ns > 1 ? part : nullptr, ns, bcorr, T, E, ng, tg, K, route_scale, idx, w);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace beam
