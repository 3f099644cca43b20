// Block-scaled (MX) expert weights for decode steps: MXFP8 and MXFP4.
//
// The pages run the routed experts in a 4-bit block format ("Reflection Beam
// 1.0 on vLLM", MoE section; the library MoE path of the optimisation
// section quantises for it). Here the experts may instead be stored in the OCP
// microscaling layouts: every 32 consecutive weights along a row's reduction
// axis share one E8M0 scale byte s (the value 2^(s - 127)).
// MXFP8: each weight is an e4m3fn code; the shared exponent of a block is
// floor(log2(amax)) - 8 (8: the exponent of the largest normal e4m3 value), so
// amax / 2^exp lies in [256, 512) and magnitudes above 448 clamp.
// MXFP4: each weight is an e2m1 code (1 sign, 2 exponent bits with bias 1, 1
// mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte (element
// 2i in the low nibble); the shared exponent is floor(log2(amax)) - 2.
//
//  mxfp8_quantize_kernel / mxfp4_quantize_kernel
//                          bf16 rows -> codes + scales, one thread per block
//  expert_w13_swiglu_mx{,4}_kernel
//                          gate/up rows of the selected experts with SwiGLU
//  expert_w2_combine_mx{,4}_kernel
//                          down projection of every selected expert and the
//                          weighted combine in fp32
// The GEMVs read 1/2 (MXFP8) or 1/4 (MXFP4) of the bytes of their bf16
// counterparts, plus 1/32 or 1/64 for the scales; codes are widened to bf16
// exactly with gfx950's packed conversions, each chunk's dot product with the
// activation is taken in fp32 and multiplied by the block's power-of-two scale.
#include "common.h"
#include "internal.h"

namespace beam {

BEAM_ERR_FLAG_DECL(mx)
BEAM_ERR_FLAG_READER(mx)

constexpr int MT = 256;  // threads per workgroup (4 waves)

// 2^(s - 127) for an E8M0 byte s (s = 0 is the binary32 subnormal 2^-127)
__device__ __forceinline__ float e8m0_value(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x400000u);
}

__device__ __forceinline__ uint4 e4m3x8_bits(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(uint4, e4m3x8_to_bf16x8(uint2{lo, hi}));
}

__global__ __launch_bounds__(MT) void mxfp8_quantize_kernel(const uint16_t* __restrict__ w,
                                                            long long nblocks,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const long long i = (long long)blockIdx.x * MT + threadIdx.x;
  if (i >= nblocks) return;
  const uint16_t* src = w + i * 32;
  uint32_t v[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 u = ld16(src + q * 8);
    v[4 * q] = u.x;
    v[4 * q + 1] = u.y;
    v[4 * q + 2] = u.z;
    v[4 * q + 3] = u.w;
  }
  // bf16 magnitudes order like their bit patterns; the exponent field of the
  // largest is floor(log2(amax)) + 127 for normal values
  uint32_t amax = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) amax = max(amax, max(v[k] & 0x7fffu, (v[k] >> 16) & 0x7fffu));
  const int eb = (int)(amax >> 7);
  const int s = eb == 0 ? -127 : max(-127, eb - 127 - 8);
  const float inv = __uint_as_float((uint32_t)(127 - s) << 23);  // 2^-s, exact scaling
  uint32_t out[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t word = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int el = 4 * k + h;  // element el: half (el & 1) of v[el >> 1]
      const uint32_t b = (el & 1) ? (v[el >> 1] & 0xffff0000u) : (v[el >> 1] << 16);
      word |= (uint32_t)f2e4m3(__uint_as_float(b) * inv) << (8 * h);
    }
    out[k] = word;
  }
  *reinterpret_cast<uint4*>(codes + i * 32) = uint4{out[0], out[1], out[2], out[3]};
  *reinterpret_cast<uint4*>(codes + i * 32 + 16) = uint4{out[4], out[5], out[6], out[7]};
  scales[i] = (uint8_t)(s + 127);
}

// Gate/up rows: workgroup (f block, slot t * topk + k); wave w takes row
// f = 4 * blockIdx.x + w of expert idx[t][k], gate row f and up row F + f,
// in 16-code chunks (lane l: chunks l, l + 64, ...). Weights and their scales
// are requested before the activation row is staged in LDS.
template <int NB>
__global__ __launch_bounds__(MT) void expert_w13_swiglu_mx_kernel(
    const uint8_t* __restrict__ w13c, const uint8_t* __restrict__ w13s,
    const int32_t* __restrict__ idx, int E, int topk, int F, int D,
    const uint16_t* __restrict__ X, uint16_t* __restrict__ act) {
  extern __shared__ __align__(16) uint16_t xs[];
  const int s = blockIdx.y;
  const int t = s / topk;
  const int e = idx[s];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int f = blockIdx.x * 4 + wave;
  if (e < 0 || e >= E) {
    if (threadIdx.x == 0 && blockIdx.x == 0) BEAM_RAISE(mx, ERR_EXPERT);
    if (lane == 0 && f < F) act[(size_t)s * F + f] = 0;
    return;
  }
  const int nc = D >> 4, nb = D >> 5;  // 16-code chunks and 32-code blocks of a row
  const size_t grow = (size_t)e * 2 * F + min(f, F - 1);
  const uint8_t* gc = w13c + grow * D;
  const uint8_t* uc = gc + (size_t)F * D;
  const uint8_t* gs = w13s + grow * nb;
  const uint8_t* us = gs + (size_t)F * nb;
  uint4 gw[NB], uw[NB];
  uint32_t gsc[NB], usc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int c = lane + 64 * b;
    const bool ok = c < nc;
    gw[b] = ok ? ld16_nt(gc + (size_t)c * 16) : uint4{0u, 0u, 0u, 0u};
    uw[b] = ok ? ld16_nt(uc + (size_t)c * 16) : uint4{0u, 0u, 0u, 0u};
    gsc[b] = ok ? gs[c >> 1] : 0u;
    usc[b] = ok ? us[c >> 1] : 0u;
  }
  for (int i = threadIdx.x; i < (D >> 3); i += MT)
    *reinterpret_cast<uint4*>(xs + i * 8) = ld16(X + (size_t)t * D + i * 8);
  __syncthreads();
  if (f >= F) return;
  float ag = 0.f, au = 0.f;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int c = lane + 64 * b;
    if (c < nc) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(xs + c * 16);
      const uint4 x1 = *reinterpret_cast<const uint4*>(xs + c * 16 + 8);
      const float pg = dot8_bf16_d2(e4m3x8_bits(gw[b].z, gw[b].w), x1,
                                 dot8_bf16_d2(e4m3x8_bits(gw[b].x, gw[b].y), x0, 0.f));
      const float pu = dot8_bf16_d2(e4m3x8_bits(uw[b].z, uw[b].w), x1,
                                 dot8_bf16_d2(e4m3x8_bits(uw[b].x, uw[b].y), x0, 0.f));
      ag = __builtin_fmaf(pg, e8m0_value(gsc[b]), ag);
      au = __builtin_fmaf(pu, e8m0_value(usc[b]), au);
    }
  }
  ag = wave_sum(ag);
  au = wave_sum(au);
  if (lane == 0) act[(size_t)s * F + f] = f2bf(siluf(round_bf(ag)) * round_bf(au));
}

// Down projection + weighted combine: workgroup (ROWS output rows, token t);
// wave w takes slots w, w + 4, ... and accumulates coef * (W2_e[row] . act)
// in 8-code chunks; the four waves' partials are added in a fixed order and
// rounded once.
template <int ROWS, int NA>
__global__ __launch_bounds__(MT) void expert_w2_combine_mx_kernel(
    const uint8_t* __restrict__ w2c, const uint8_t* __restrict__ w2s,
    const int32_t* __restrict__ idx, const float* __restrict__ wts, int E, int topk, int F,
    int D, const uint16_t* __restrict__ act, uint16_t* __restrict__ Y) {
  __shared__ float part[4][ROWS];
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d0 = blockIdx.x * ROWS;
  const int nc = F >> 3, nb = F >> 5;
  float accr[ROWS] = {};
  for (int k = wave; k < topk; k += 4) {
    const int e = idx[t * topk + k];
    if (e < 0 || e >= E) {
      if (lane == 0 && blockIdx.x == 0) BEAM_RAISE(mx, ERR_EXPERT);
      continue;
    }
    const uint8_t* wb = w2c + (size_t)e * D * F;
    const uint8_t* sb = w2s + (size_t)e * D * nb;
    const uint16_t* ab = act + ((size_t)t * topk + k) * F;
    const float coef = wts[t * topk + k];
    uint2 wv[ROWS][NA];
    uint32_t sc[ROWS][NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = lane + 64 * i;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const bool ok = c < nc && d0 + r < D;
        wv[r][i] = ok ? *reinterpret_cast<const uint2*>(wb + (size_t)(d0 + r) * F + (size_t)c * 8)
                      : uint2{0u, 0u};
        sc[r][i] = ok ? sb[(size_t)(d0 + r) * nb + (c >> 2)] : 0u;
      }
    }
    uint4 av[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = lane + 64 * i;
      av[i] = c < nc ? ld16(ab + (size_t)c * 8) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < NA; ++i)
        a = __builtin_fmaf(dot8_bf16_d2(e4m3x8_bits(wv[r][i].x, wv[r][i].y), av[i], 0.f),
                           e8m0_value(sc[r][i]), a);
      accr[r] = __builtin_fmaf(coef, a, accr[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) accr[r] = wave_sum(accr[r]);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) part[wave][r] = accr[r];
  }
  __syncthreads();
  if (threadIdx.x < ROWS && d0 + (int)threadIdx.x < D) {
    const int r = threadIdx.x;
    const float v = ((part[0][r] + part[1][r]) + part[2][r]) + part[3][r];
    Y[(size_t)t * D + d0 + r] = f2bf(v);
  }
}

// ---- MXFP4 -------------------------------------------------------------------
// e2m1 code of a scaled weight: the magnitude code counts the midpoints between
// consecutive e2m1 values that lie below |x| (on a midpoint the even code wins:
// strict comparisons at midpoints below an even code, non-strict below an odd
// one), saturating at 6; the sign bit is copied (so -0 keeps it).
__device__ __forceinline__ uint32_t f2e2m1(float x) {
  const float a = fabsf(x);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

// Eight e2m1 codes of a word -> eight bf16 (exact, unit scale); byte b holds
// elements 2b (low nibble) and 2b + 1.
__device__ __forceinline__ uint4 e2m1x8_bits(uint32_t w) {
  return uint4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3))};
}

__global__ __launch_bounds__(MT) void mxfp4_quantize_kernel(const uint16_t* __restrict__ w,
                                                            long long nblocks,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const long long i = (long long)blockIdx.x * MT + threadIdx.x;
  if (i >= nblocks) return;
  const uint16_t* src = w + i * 32;
  uint32_t v[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 u = ld16(src + q * 8);
    v[4 * q] = u.x;
    v[4 * q + 1] = u.y;
    v[4 * q + 2] = u.z;
    v[4 * q + 3] = u.w;
  }
  uint32_t amax = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) amax = max(amax, max(v[k] & 0x7fffu, (v[k] >> 16) & 0x7fffu));
  const int eb = (int)(amax >> 7);
  const int s = eb == 0 ? -127 : max(-127, eb - 127 - 2);
  const float inv = __uint_as_float((uint32_t)(127 - s) << 23);  // 2^-s, exact scaling
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // word k: elements 8k .. 8k + 7, nibble n = element 8k + n
    uint32_t word = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int el = 8 * k + n;
      const uint32_t b = (el & 1) ? (v[el >> 1] & 0xffff0000u) : (v[el >> 1] << 16);
      word |= f2e2m1(__uint_as_float(b) * inv) << (4 * n);
    }
    out[k] = word;
  }
  *reinterpret_cast<uint4*>(codes + i * 16) = uint4{out[0], out[1], out[2], out[3]};
  scales[i] = (uint8_t)(s + 127);
}

// MXFP4 rows are read in 16-byte chunks of 32 codes: exactly one scaled
// block, so chunk c of a row has scale byte c, and one wave instruction
// covers 1 KiB of codes. A lane's chunk meets 32 activations (64 bytes); in
// LDS the four 16-byte pieces q of activation chunk c sit at slot
// 4 c + (q ^ ((c >> 2) & 3)), so the 16 lanes served per LDS cycle (chunks
// c .. c + 15, one piece each) hit 16 distinct slots of the 64 banks.
__device__ __forceinline__ int mx4_xslot(int c, int q) { return 4 * c + (q ^ ((c >> 2) & 3)); }

__device__ __forceinline__ float mx4_chunk_dot(uint4 w, const uint4 (&x)[4], float acc) {
  acc = dot8_bf16_d2(e2m1x8_bits(w.x), x[0], acc);
  acc = dot8_bf16_d2(e2m1x8_bits(w.y), x[1], acc);
  acc = dot8_bf16_d2(e2m1x8_bits(w.z), x[2], acc);
  return dot8_bf16_d2(e2m1x8_bits(w.w), x[3], acc);
}

// Gate/up rows, MXFP4, with SwiGLU: wave w takes rows
// f0 = NR * (4 * blockIdx.x + w) .. + NR - 1 of the expert of slot s; every
// code and scale load of the wave is in flight before the activation is
// staged.
template <int NB, int NR>
__global__ __launch_bounds__(MT) void expert_w13_swiglu_mx4_kernel(
    const uint8_t* __restrict__ w13c, const uint8_t* __restrict__ w13s,
    const int32_t* __restrict__ idx, int E, int topk, int F, int D,
    const uint16_t* __restrict__ X, uint16_t* __restrict__ act) {
  extern __shared__ __align__(16) uint16_t xs[];
  const int s = blockIdx.y;
  const int t = s / topk;
  const int e = idx[s];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int f0 = (blockIdx.x * 4 + wave) * NR;
  if (e < 0 || e >= E) {  // uniform over the workgroup
    if (threadIdx.x == 0 && blockIdx.x == 0) BEAM_RAISE(mx, ERR_EXPERT);
    if (lane < NR && f0 + lane < F) act[(size_t)s * F + f0 + lane] = 0;
    return;
  }
  const int nch = D >> 5;            // 32-code chunks (scaled blocks) of a row
  const size_t rb = (size_t)D >> 1;  // bytes of a row
  uint4 gw[NR][NB], uw[NR][NB];
  uint32_t gsc[NR][NB], usc[NR][NB];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const size_t grow = (size_t)e * 2 * F + min(f0 + r, F - 1);
    const uint8_t* gc = w13c + grow * rb;
    const uint8_t* uc = gc + (size_t)F * rb;
    const uint8_t* gs = w13s + grow * nch;
    const uint8_t* us = gs + (size_t)F * nch;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c = min(lane + 64 * b, nch - 1);  // past the row: re-read, left out below
      gw[r][b] = ld16_nt(gc + (size_t)c * 16);
      uw[r][b] = ld16_nt(uc + (size_t)c * 16);
      gsc[r][b] = gs[c];
      usc[r][b] = us[c];
    }
  }
  for (int i = threadIdx.x; i < (D >> 3); i += MT)
    *reinterpret_cast<uint4*>(xs + mx4_xslot(i >> 2, i & 3) * 8) =
        ld16(X + (size_t)t * D + i * 8);
  __syncthreads();
  float ag[NR] = {}, au[NR] = {};
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int c = lane + 64 * b;
    if (c < nch) {
      uint4 x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = *reinterpret_cast<const uint4*>(xs + mx4_xslot(c, q) * 8);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        ag[r] = __builtin_fmaf(mx4_chunk_dot(gw[r][b], x, 0.f), e8m0_value(gsc[r][b]), ag[r]);
        au[r] = __builtin_fmaf(mx4_chunk_dot(uw[r][b], x, 0.f), e8m0_value(usc[r][b]), au[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float g = wave_sum(ag[r]), u = wave_sum(au[r]);
    if (lane == 0 && f0 + r < F) act[(size_t)s * F + f0 + r] = f2bf(siluf(round_bf(g)) * round_bf(u));
  }
}

// Down projection + weighted combine, MXFP4: ROWS output rows per workgroup
// and NW waves, wave w taking slots w, w + NW, ... (one each when topk <= NW,
// so every weight load of the workgroup is in flight at once); a slot's
// activation chunk (64 bytes per lane, straight from global memory) serves
// all ROWS rows. The waves' partials are added in a fixed order.
template <int ROWS, int NA, int NW>
__global__ __launch_bounds__(NW * 64) void expert_w2_combine_mx4_kernel(
    const uint8_t* __restrict__ w2c, const uint8_t* __restrict__ w2s,
    const int32_t* __restrict__ idx, const float* __restrict__ wts, int E, int topk, int F,
    int D, const uint16_t* __restrict__ act, uint16_t* __restrict__ Y) {
  __shared__ float part[NW][ROWS];
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d0 = blockIdx.x * ROWS;
  const int nch = F >> 5;
  const size_t rb = (size_t)F >> 1;
  float accr[ROWS] = {};
  for (int k = wave; k < topk; k += NW) {
    const int e = idx[t * topk + k];
    if (e < 0 || e >= E) {
      if (lane == 0 && blockIdx.x == 0) BEAM_RAISE(mx, ERR_EXPERT);
      continue;
    }
    const uint8_t* wb = w2c + (size_t)e * D * rb;
    const uint8_t* sb = w2s + (size_t)e * D * nch;
    const uint16_t* ab = act + ((size_t)t * topk + k) * F;
    const float coef = wts[t * topk + k];
    uint4 wv[ROWS][NA];
    uint32_t sc[ROWS][NA];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const int row = min(d0 + r, D - 1);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int c = min(lane + 64 * i, nch - 1);  // past the row: re-read, left out below
        wv[r][i] = ld16_nt(wb + (size_t)row * rb + (size_t)c * 16);
        sc[r][i] = sb[(size_t)row * nch + c];
      }
    }
    uint4 av[NA][4];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = min(lane + 64 * i, nch - 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) av[i][q] = ld16(ab + (size_t)c * 32 + q * 8);
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < NA; ++i)
        if (lane + 64 * i < nch)
          a = __builtin_fmaf(mx4_chunk_dot(wv[r][i], av[i], 0.f), e8m0_value(sc[r][i]), a);
      accr[r] = __builtin_fmaf(coef, a, accr[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) accr[r] = wave_sum(accr[r]);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) part[wave][r] = accr[r];
  }
  __syncthreads();
  if (threadIdx.x < ROWS && d0 + (int)threadIdx.x < D) {
    const int r = threadIdx.x;
    float v = part[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += part[w][r];
    Y[(size_t)t * D + d0 + r] = f2bf(v);
  }
}

#define LAUNCH_OK() (hipGetLastError() == hipSuccess ? 0 : -1)

int launch_mxfp8_quantize(const uint16_t* w, long long nblocks, uint8_t* codes, uint8_t* scales,
                          hipStream_t st) {
  hipLaunchKernelGGL(mxfp8_quantize_kernel, dim3((unsigned)((nblocks + MT - 1) / MT)), dim3(MT),
                     0, st, w, nblocks, codes, scales);
  return LAUNCH_OK();
}

// act: [T * topk][F] bf16 scratch.
int launch_moe_mxfp8(int T, int D, int F, int E, int topk, const uint8_t* w13c,
                     const uint8_t* w13s, const uint8_t* w2c, const uint8_t* w2s,
                     const int32_t* idx, const float* wts, const uint16_t* X, uint16_t* act,
                     uint16_t* Y, hipStream_t st) {
  const int nc13 = D / 16, nc2 = F / 8;
  const dim3 g13((F + 3) / 4, T * topk);
  const size_t sh = (size_t)D * 2;
  if (nc13 <= 64)
    hipLaunchKernelGGL((expert_w13_swiglu_mx_kernel<1>), g13, dim3(MT), sh, st, w13c, w13s, idx,
                       E, topk, F, D, X, act);
  else if (nc13 <= 64 * 5)
    hipLaunchKernelGGL((expert_w13_swiglu_mx_kernel<5>), g13, dim3(MT), sh, st, w13c, w13s, idx,
                       E, topk, F, D, X, act);
  else
    return -2;
  if (hipGetLastError() != hipSuccess) return -1;
  constexpr int ROWS = 2;
  const dim3 g2((D + ROWS - 1) / ROWS, T);
  if (nc2 <= 64)
    hipLaunchKernelGGL((expert_w2_combine_mx_kernel<ROWS, 1>), g2, dim3(MT), 0, st, w2c, w2s, idx,
                       wts, E, topk, F, D, act, Y);
  else if (nc2 <= 64 * 5)
    hipLaunchKernelGGL((expert_w2_combine_mx_kernel<ROWS, 5>), g2, dim3(MT), 0, st, w2c, w2s, idx,
                       wts, E, topk, F, D, act, Y);
  else
    return -2;
  return LAUNCH_OK();
}

int launch_mxfp4_quantize(const uint16_t* w, long long nblocks, uint8_t* codes, uint8_t* scales,
                          hipStream_t st) {
  hipLaunchKernelGGL(mxfp4_quantize_kernel, dim3((unsigned)((nblocks + MT - 1) / MT)), dim3(MT),
                     0, st, w, nblocks, codes, scales);
  return LAUNCH_OK();
}

// act: [T * topk][F] bf16 scratch.
int launch_moe_mxfp4(int T, int D, int F, int E, int topk, const uint8_t* w13c,
                     const uint8_t* w13s, const uint8_t* w2c, const uint8_t* w2s,
                     const int32_t* idx, const float* wts, const uint16_t* X, uint16_t* act,
                     uint16_t* Y, hipStream_t st) {
  // measured best on MI355X at Beam's shapes (more rows per wave, or more
  // waves per down-projection workgroup, ran slower); NW: waves of the
  // down-projection workgroup
  constexpr int NR = 2, ROWS = 4, NW = 4;
  const int nch13 = D / 32, nch2 = F / 32;  // 32-code chunks
  if (nch13 > 64 * 3 || nch2 > 64 * 2) return -2;
  const dim3 g13((F + 4 * NR - 1) / (4 * NR), T * topk);
  const size_t sh = (size_t)D * 2;
  if (nch13 <= 64)
    hipLaunchKernelGGL((expert_w13_swiglu_mx4_kernel<1, NR>), g13, dim3(MT), sh, st, w13c, w13s,
                       idx, E, topk, F, D, X, act);
  else
    hipLaunchKernelGGL((expert_w13_swiglu_mx4_kernel<3, NR>), g13, dim3(MT), sh, st, w13c, w13s,
                       idx, E, topk, F, D, X, act);
  if (hipGetLastError() != hipSuccess) return -1;
  const dim3 g2((D + ROWS - 1) / ROWS, T);
  if (nch2 <= 64)
    hipLaunchKernelGGL((expert_w2_combine_mx4_kernel<ROWS, 1, NW>), g2, dim3(NW * 64), 0, st,
                       w2c, w2s, idx, wts, E, topk, F, D, act, Y);
  else
    hipLaunchKernelGGL((expert_w2_combine_mx4_kernel<ROWS, 2, NW>), g2, dim3(NW * 64), 0, st,
                       w2c, w2s, idx, wts, E, topk, F, D, act, Y);
  return LAUNCH_OK();
}

}  // namespace beam
