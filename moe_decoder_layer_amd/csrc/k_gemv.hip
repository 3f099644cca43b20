// Weight-streaming GEMV kernels for few-token (decode) steps.
//
// At batch 1 every projection is bound by reading its bf16 weight once from
// HBM. Each wave owns R weight rows and streams them with 16-byte
// non-temporal loads (lane l reads chunks l, l+64, ...: every load
// instruction covers 1 KiB of contiguous row), NB chunks per row in flight
// per batch. The activation rows are staged once per workgroup in LDS and
// read back with conflict-free 16-byte LDS reads. Sums are fp32, reduced
// across the wave with xor shuffles; results are rounded to bf16 once.
//
//  gemv_qkvg_kernel    packed q|k|v|gate projection ("Reflection Beam 1.0 on
//                      vLLM", optimisation change 5); q|k|v rows go to a
//                      workspace for the per-head epilogue, gate rows straight
//                      to their output
//  gemv_gate_oproj     sigmoid output gate fused as the prologue of o_proj
//                      (Attention section; change 2's gate kernel)
//  expert_w13_swiglu   gate and up rows of the routed experts with the SwiGLU
//                      epilogue (MoE section); only the selected experts'
//                      rows are read (the small-batch MoE kernels of the
//                      Flint page, optimisation strategy section)
//  expert_w2_combine   down projection of every selected expert and the
//                      weighted combine in fp32 (optimisation change 3)
#include "common.h"
#include "internal.h"

namespace beam {

BEAM_ERR_FLAG_DECL(gemv)
BEAM_ERR_FLAG_READER(gemv)

constexpr int GT = 256;  // threads per workgroup (4 waves)

// Copy `rows` activation rows of K bf16 into LDS (zero rows beyond `valid`).
__device__ __forceinline__ void stage_rows(uint16_t* xs, const uint16_t* __restrict__ X,
                                           size_t ldx, int K, int rows, int valid) {
  const int nc = K >> 3;
  for (int i = threadIdx.x; i < rows * nc; i += GT) {
    const int r = i / nc, c = i - r * nc;
    uint4 v = {0u, 0u, 0u, 0u};
    if (r < valid) v = ld16(X + (size_t)r * ldx + c * 8);
    *reinterpret_cast<uint4*>(xs + (size_t)r * K + c * 8) = v;
  }
}

// acc[r][t] += W[row r] . xs[t] for R rows, TT activation rows in LDS.
template <int R, int NB, int TT>
__device__ __forceinline__ void rows_dot(const uint16_t* const (&wr)[R], int K,
                                         const uint16_t* xs, int lane, float (&acc)[R][TT]) {
  const int nc = K >> 3;
  for (int c0 = 0; c0 < nc; c0 += 64 * NB) {
    uint4 wv[R][NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c = c0 + lane + 64 * b;
#pragma unroll
      for (int r = 0; r < R; ++r)
        wv[r][b] = (c < nc && wr[r]) ? ld16_nt(wr[r] + (size_t)c * 8) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c = c0 + lane + 64 * b;
      if (c < nc) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const uint4 xv = *reinterpret_cast<const uint4*>(xs + (size_t)t * K + c * 8);
#pragma unroll
          for (int r = 0; r < R; ++r) acc[r][t] = dot8_bf16(wv[r][b], xv, acc[r][t]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[r][t] = wave_sum(acc[r][t]);
}

// ---------------------------------------------------------------------------
// Packed q|k|v|gate projection. Rows [0, Nqkv) -> qkv[t][row], rows
// [Nqkv, N) -> g_out[t][row - Nqkv].
template <int R, int NB, int TT>
__global__ __launch_bounds__(GT) void gemv_qkvg_kernel(const uint16_t* __restrict__ W, int N,
                                                       int K, const uint16_t* __restrict__ X,
                                                       int T, int Nqkv,
                                                       uint16_t* __restrict__ qkv,
                                                       uint16_t* __restrict__ g_out) {
  extern __shared__ __align__(16) uint16_t xs[];
  const int t0 = blockIdx.y * TT;
  stage_rows(xs, X + (size_t)t0 * K, K, K, TT, min(TT, T - t0));
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * R;
  if (n0 >= N) return;
  const uint16_t* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = (n0 + r < N) ? W + (size_t)(n0 + r) * K : nullptr;
  float acc[R][TT] = {};
  rows_dot<R, NB, TT>(wr, K, xs, lane, acc);
  if (lane == 0) {
    const int G = N - Nqkv;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = n0 + r;
      if (n >= N) break;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        if (t0 + t >= T) break;
        const uint16_t v = f2bf(acc[r][t]);
        if (n < Nqkv) qkv[(size_t)(t0 + t) * Nqkv + n] = v;
        else g_out[(size_t)(t0 + t) * G + (n - Nqkv)] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// o_proj with the output gate as prologue: z = bf16(o * sigmoid(g + b[head]))
// is formed in LDS, then y[t][n] = bf16(W_o[n] . z[t]).
template <int R, int NB, int TT>
__global__ __launch_bounds__(GT) void gemv_gate_oproj_kernel(
    const uint16_t* __restrict__ W, int N, int K, const uint16_t* __restrict__ O,
    const uint16_t* __restrict__ Gt, const uint16_t* __restrict__ bgate, int hd, int T,
    uint16_t* __restrict__ Y) {
  extern __shared__ __align__(16) uint16_t xs[];
  const int t0 = blockIdx.y * TT;
  const int nc = K >> 3;
  for (int i = threadIdx.x; i < TT * nc; i += GT) {
    const int r = i / nc, c = i - r * nc;
    uint4 z = {0u, 0u, 0u, 0u};
    if (t0 + r < T) {
      const size_t off = (size_t)(t0 + r) * K + c * 8;
      z = ld16(O + off);
      if (Gt) {
        const uint4 gv = ld16(Gt + off);
        const float b = bf2f(bgate[(c * 8) / hd]);  // 8-chunks never straddle heads
        const uint32_t* zi = reinterpret_cast<const uint32_t*>(&z);
        const uint32_t* gi = reinterpret_cast<const uint32_t*>(&gv);
        uint32_t out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a0 = bf_lo(zi[e]) * sigmoidf_fast(bf_lo(gi[e]) + b);
          const float a1 = bf_hi(zi[e]) * sigmoidf_fast(bf_hi(gi[e]) + b);
          out[e] = pack_bf2(a0, a1);
        }
        z = uint4{out[0], out[1], out[2], out[3]};
      }
    }
    *reinterpret_cast<uint4*>(xs + (size_t)r * K + c * 8) = z;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * R;
  if (n0 >= N) return;
  const uint16_t* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = (n0 + r < N) ? W + (size_t)(n0 + r) * K : nullptr;
  float acc[R][TT] = {};
  rows_dot<R, NB, TT>(wr, K, xs, lane, acc);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (n0 + r >= N) break;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        if (t0 + t >= T) break;
        Y[(size_t)(t0 + t) * N + n0 + r] = f2bf(acc[r][t]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Single-token packed projection, a grid resident all at once: each wave
// requests its whole weight row (NB chunks per lane, K = 64 * NB * 8) before
// the workgroup stages the activation, so the HBM stream starts at once
// instead of after the staging round trip.
template <int NB>
__global__ __launch_bounds__(GT) void gemv_qkvg_wf_kernel(const uint16_t* __restrict__ W, int N,
                                                          int K, const uint16_t* __restrict__ X,
                                                          int Nqkv, uint16_t* __restrict__ qkv,
                                                          uint16_t* __restrict__ g_out) {
  extern __shared__ __align__(16) uint16_t xs[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + wave;
  const uint16_t* wr = W + (size_t)min(n, N - 1) * K;
  uint4 wv[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) wv[b] = ld16_nt(wr + (size_t)(lane + 64 * b) * 8);
  stage_rows(xs, X, K, K, 1, 1);
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int b = 0; b < NB; ++b)
    acc = dot8_bf16(wv[b], *reinterpret_cast<const uint4*>(xs + (lane + 64 * b) * 8), acc);
  acc = wave_sum(acc);
  if (lane == 0 && n < N) {
    const uint16_t v = f2bf(acc);
    if (n < Nqkv) qkv[n] = v;
    else g_out[n - Nqkv] = v;
  }
}

// ---------------------------------------------------------------------------
// Expert gate/up rows with SwiGLU. Slot s = t * spt + k (spt = topk, plus one
// for a shared expert): expert e = idx[t*topk + k] (k < topk) or the shared
// expert (k == topk). act[s][f] = bf16(silu(bf16(gate_f . x)) * bf16(up_f . x)).
// idx == nullptr: a single dense "expert" at w13 (spt = 1).
template <int P, int NB>
__global__ __launch_bounds__(GT) void expert_w13_swiglu_kernel(
    const uint16_t* __restrict__ w13, const uint16_t* __restrict__ shared_w13,
    const int32_t* __restrict__ idx, int E, int topk, int spt, int F, int D,
    const uint16_t* __restrict__ X, uint16_t* __restrict__ act) {
  extern __shared__ __align__(16) uint16_t xs[];
  const int s = blockIdx.y;
  const int t = s / spt, k = s - t * spt;
  const uint16_t* base;
  if (idx == nullptr) {
    base = w13;
  } else if (k < topk) {
    const int e = idx[t * topk + k];
    if (e < 0 || e >= E) {
      if (threadIdx.x == 0 && blockIdx.x == 0) BEAM_RAISE(gemv, ERR_EXPERT);
      for (int f = blockIdx.x * 4 * P + threadIdx.x; f < min(F, (blockIdx.x + 1) * 4 * P);
           f += GT)
        act[(size_t)s * F + f] = 0;
      return;
    }
    base = w13 + (size_t)e * 2 * F * D;
  } else {
    base = shared_w13;
  }
  stage_rows(xs, X + (size_t)t * D, D, D, 1, 1);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int f0 = (blockIdx.x * 4 + wave) * P;
  if (f0 >= F) return;
  const uint16_t* wr[2 * P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const bool ok = f0 + p < F;
    wr[p] = ok ? base + (size_t)(f0 + p) * D : nullptr;
    wr[P + p] = ok ? base + (size_t)(F + f0 + p) * D : nullptr;
  }
  float acc[2 * P][1] = {};
  rows_dot<2 * P, NB, 1>(wr, D, xs, lane, acc);
  if (lane == 0) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (f0 + p >= F) break;
      const float gt = round_bf(acc[p][0]), up = round_bf(acc[P + p][0]);
      act[(size_t)s * F + f0 + p] = f2bf(siluf(gt) * up);
    }
  }
}

// ---------------------------------------------------------------------------
// Down projection + weighted combine. Each workgroup owns ROWS output rows of
// one token; wave w takes slots w, w+4, ... and accumulates
// coef_slot * (W2_slot[row] . act_slot) per row; the four waves' partials are
// summed in a fixed order (deterministic, no atomics) and rounded once.
// MoE: slots k < topk use expert idx[t][k] with coef w[t][k]; slot topk (if
// shared_w2) uses the shared expert with coef 1.  Dense (idx == nullptr): the
// d_ff axis is cut into 8 slices of F/8 treated as slots with coef 1.
template <int ROWS, int NA>
__global__ __launch_bounds__(GT) void expert_w2_combine_kernel(
    const uint16_t* __restrict__ w2, const uint16_t* __restrict__ shared_w2,
    const int32_t* __restrict__ idx, const float* __restrict__ wts, int E, int topk, int spt,
    int F, int D, const uint16_t* __restrict__ act, uint16_t* __restrict__ Y) {
  __shared__ float part[4][ROWS];
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d0 = blockIdx.x * ROWS;
  const bool dense = (idx == nullptr);
  const int nslots = dense ? 8 : spt;
  const int Ks = dense ? F / 8 : F;
  const int nca = Ks >> 3;
  float accr[ROWS] = {};
  for (int s = wave; s < nslots; s += 4) {
    const uint16_t* wb;
    const uint16_t* ab;
    float coef;
    if (dense) {
      wb = w2 + (size_t)s * Ks;
      ab = act + (size_t)t * F + (size_t)s * Ks;
      coef = 1.f;
    } else if (s < topk) {
      const int e = idx[t * topk + s];
      if (e < 0 || e >= E) {
        if (lane == 0 && blockIdx.x == 0) BEAM_RAISE(gemv, ERR_EXPERT);
        continue;
      }
      wb = w2 + (size_t)e * D * F;
      ab = act + ((size_t)t * spt + s) * F;
      coef = wts[t * topk + s];
    } else {
      wb = shared_w2;
      ab = act + ((size_t)t * spt + s) * F;
      coef = 1.f;
    }
    uint4 av[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int c = lane + 64 * i;
      av[i] = (c < nca) ? ld16(ab + c * 8) : uint4{0u, 0u, 0u, 0u};
    }
    for (int c0 = 0; c0 < nca; c0 += 64 * NA) {
      uint4 wv[ROWS][NA];
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int c = c0 + lane + 64 * i;
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
          wv[r][i] = (c < nca && d0 + r < D)
                         ? ld16_nt(wb + (size_t)(d0 + r) * F + (size_t)c * 8)
                         : uint4{0u, 0u, 0u, 0u};
      }
      if (c0 > 0) {
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          const int c = c0 + lane + 64 * i;
          av[i] = (c < nca) ? ld16(ab + c * 8) : uint4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < NA; ++i) a = dot8_bf16(wv[r][i], av[i], a);
        accr[r] = __builtin_fmaf(coef, a, accr[r]);
      }
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

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Output head with the logit soft cap (Beam's architecture notes): logits
// [T][V] fp32 = cap * tanh((x . W[v]) / cap), or x . W[v] when cap is 0.
__device__ __forceinline__ float softcap_f(float z, float cap) {
  return cap > 0.f ? cap * tanhf(z / cap) : z;
}

template <int R, int NB, int TT>
__global__ __launch_bounds__(GT) void gemv_lm_head_kernel(const uint16_t* __restrict__ W, int V,
                                                          int K, const uint16_t* __restrict__ X,
                                                          int T, float cap,
                                                          float* __restrict__ logits) {
  extern __shared__ __align__(16) uint16_t xs[];
  const int t0 = blockIdx.y * TT;
  stage_rows(xs, X + (size_t)t0 * K, K, K, TT, min(TT, T - t0));
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * R;
  if (n0 >= V) return;
  const uint16_t* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = (n0 + r < V) ? W + (size_t)(n0 + r) * K : nullptr;
  float acc[R][TT] = {};
  rows_dot<R, NB, TT>(wr, K, xs, lane, acc);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (n0 + r >= V) break;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        if (t0 + t >= T) break;
        logits[(size_t)(t0 + t) * V + n0 + r] = softcap_f(acc[r][t], cap);
      }
    }
  }
}

// In-place soft cap over n fp32 logits (after the many-token GEMM).
__global__ __launch_bounds__(GT) void softcap_kernel(float* __restrict__ z, long long n,
                                                     float cap) {
  const long long i = (long long)blockIdx.x * GT + threadIdx.x;
  if (i < n) z[i] = softcap_f(z[i], cap);
}

int launch_softcap(float* z, long long n, float cap, hipStream_t st) {
  hipLaunchKernelGGL(softcap_kernel, dim3((unsigned)((n + GT - 1) / GT)), dim3(GT), 0, st, z, n,
                     cap);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// launchers
static int nb_for(int nc) {
  if (nc % 640 == 0) return 10;
  if (nc % 384 == 0) return 6;
  if (nc % 320 == 0) return 5;
  return 4;
}

#define LAUNCH_OK() (hipGetLastError() == hipSuccess ? 0 : -1)

int launch_gemv_qkvg(int T, int N, int K, int Nqkv, const uint16_t* W, const uint16_t* X,
                     uint16_t* qkv, uint16_t* g_out, hipStream_t st) {
  constexpr int R = 2;
  const dim3 grid((N + 4 * R - 1) / (4 * R), 1);
  const int nb = nb_for(K >> 3);
  if (T == 1 && (K >> 3) == 640) {
    hipLaunchKernelGGL((gemv_qkvg_wf_kernel<10>), dim3((N + 3) / 4), dim3(GT), (size_t)K * 2, st,
                       W, N, K, X, Nqkv, qkv, g_out);
    return LAUNCH_OK();
  }
  if (T == 1) {
    const size_t sh = (size_t)K * 2;
#define Q1(NB) hipLaunchKernelGGL((gemv_qkvg_kernel<R, NB, 1>), grid, dim3(GT), sh, st, W, N, K, X, T, Nqkv, qkv, g_out)
    if (nb == 10) Q1(10); else if (nb == 6) Q1(6); else if (nb == 5) Q1(5); else Q1(4);
#undef Q1
  } else {
    const size_t sh = (size_t)K * 2 * 4;
    const dim3 g4(grid.x, (T + 3) / 4);
    hipLaunchKernelGGL((gemv_qkvg_kernel<R, 4, 4>), g4, dim3(GT), sh, st, W, N, K, X, T, Nqkv,
                       qkv, g_out);
  }
  return LAUNCH_OK();
}

int launch_gemv_lm_head(int T, int V, int K, const uint16_t* W, const uint16_t* X, float cap,
                        float* logits, hipStream_t st) {
  constexpr int R = 2;
  const dim3 grid((V + 4 * R - 1) / (4 * R), 1);
  if (T == 1) {
    const size_t sh = (size_t)K * 2;
    const int nb = nb_for(K >> 3);
#define H1(NB) hipLaunchKernelGGL((gemv_lm_head_kernel<R, NB, 1>), grid, dim3(GT), sh, st, W, V, K, X, T, cap, logits)
    if (nb == 10) H1(10); else if (nb == 6) H1(6); else if (nb == 5) H1(5); else H1(4);
#undef H1
  } else {
    const size_t sh = (size_t)K * 2 * 4;
    const dim3 g4(grid.x, (T + 3) / 4);
    hipLaunchKernelGGL((gemv_lm_head_kernel<R, 4, 4>), g4, dim3(GT), sh, st, W, V, K, X, T, cap,
                       logits);
  }
  return LAUNCH_OK();
}

int launch_gemv_gate_oproj(int T, int N, int K, int hd, const uint16_t* W, const uint16_t* O,
                           const uint16_t* G, const uint16_t* bgate, uint16_t* Y,
                           hipStream_t st) {
  constexpr int R = 1;
  const dim3 grid((N + 4 * R - 1) / (4 * R), 1);
  if (T == 1 && G == nullptr && (K & 511) == 0) {
    // no gate prologue: the weights-first GEMV (each wave's whole row in
    // flight before the activation is staged)
    const int nb = K >> 9;  // 16-byte chunks per lane
    const dim3 g1((N + 3) / 4);
    const size_t sh = (size_t)K * 2;
#define WF(NB) hipLaunchKernelGGL((gemv_qkvg_wf_kernel<NB>), g1, dim3(GT), sh, st, W, N, K, O, N, Y, nullptr)
    if (nb == 12) { WF(12); return LAUNCH_OK(); }
    if (nb == 10) { WF(10); return LAUNCH_OK(); }
    if (nb == 8) { WF(8); return LAUNCH_OK(); }
    if (nb == 4) { WF(4); return LAUNCH_OK(); }
#undef WF
  }
  if (T == 1) {
    const size_t sh = (size_t)K * 2;
    const int nb = nb_for(K >> 3);
#define O1(NB) hipLaunchKernelGGL((gemv_gate_oproj_kernel<R, NB, 1>), grid, dim3(GT), sh, st, W, N, K, O, G, bgate, hd, T, Y)
    if (nb == 10) O1(10); else if (nb == 6) O1(6); else if (nb == 5) O1(5); else O1(4);
#undef O1
  } else {
    const size_t sh = (size_t)K * 2 * 4;
    const dim3 g4(grid.x, (T + 3) / 4);
    hipLaunchKernelGGL((gemv_gate_oproj_kernel<R, 4, 4>), g4, dim3(GT), sh, st, W, N, K, O, G,
                       bgate, hd, T, Y);
  }
  return LAUNCH_OK();
}

int launch_expert_w13(int T, int D, int F, int E, int topk, int spt, const uint16_t* w13,
                      const uint16_t* shared_w13, const int32_t* idx, const uint16_t* X,
                      uint16_t* act, hipStream_t st) {
  constexpr int P = 1;
  const dim3 grid((F + 4 * P - 1) / (4 * P), T * spt);
  const size_t sh = (size_t)D * 2;
  const int nb = nb_for(D >> 3);
#define W13(NB) hipLaunchKernelGGL((expert_w13_swiglu_kernel<P, NB>), grid, dim3(GT), sh, st, w13, shared_w13, idx, E, topk, spt, F, D, X, act)
  if (nb == 10) W13(10); else if (nb == 6) W13(6); else if (nb == 5) W13(5); else W13(4);
#undef W13
  return LAUNCH_OK();
}

int launch_expert_w2(int T, int D, int F, int E, int topk, int spt, const uint16_t* w2,
                     const uint16_t* shared_w2, const int32_t* idx, const float* wts,
                     const uint16_t* act, uint16_t* Y, hipStream_t st) {
  constexpr int ROWS = 2;
  const dim3 grid((D + ROWS - 1) / ROWS, T);
  const int Ks = idx ? F : F / 8;
  const int nca = Ks >> 3;
  if (nca <= 64 * 5 && nca % 320 == 0)
    hipLaunchKernelGGL((expert_w2_combine_kernel<ROWS, 5>), grid, dim3(GT), 0, st, w2,
                       shared_w2, idx, wts, E, topk, spt, F, D, act, Y);
  else
    hipLaunchKernelGGL((expert_w2_combine_kernel<ROWS, 4>), grid, dim3(GT), 0, st, w2,
                       shared_w2, idx, wts, E, topk, spt, F, D, act, Y);
  return LAUNCH_OK();
}

}  // namespace beam
