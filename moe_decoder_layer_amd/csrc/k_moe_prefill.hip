// Many-token expert dispatch for the routed SwiGLU experts ("Reflection Beam
// 1.0 on vLLM", MoE section: every token goes to its 8 selected experts; the
// page's decode graph uses two routing kernels and two grouped GEMMs).
//
//   moe_count_kernel    one workgroup per expert counts its (token, slot) pairs
//   moe_scan_kernel     row offsets of the expert segments and prefix sums of
//                       their GEMM tile counts
//   moe_scatter_kernel  one workgroup per expert writes its pairs in (token,
//                       slot) order: perm[row] = token, inv[token * K + slot] = row
//   moe_combine_kernel  y[t] = bf16(sum_k w[t][k] * out[inv[t][k]] (+ shared))
// All integer work is deterministic (no atomics, stable order), so the grouped
// GEMM rows and the combine order are the same on every run.
// gate_kernel forms z = bf16(o * sigmoid(g + b[head])) for the o_proj GEMM.
#include "common.h"
#include "internal.h"

namespace beam {

BEAM_ERR_FLAG_DECL(moe)
BEAM_ERR_FLAG_READER(moe)

__device__ __forceinline__ int block_sum_int(int v, int* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void moe_count_kernel(const int32_t* __restrict__ idx, int P,
                                                        int E, int32_t* __restrict__ counts) {
  __shared__ int red[4];
  const int e = blockIdx.x;
  int c = 0;
  for (int i = threadIdx.x; i < P; i += 256) {
    const int v = idx[i];
    c += (v == e);
    if (e == 0 && (v < 0 || v >= E)) BEAM_RAISE(moe, ERR_EXPERT);
  }
  c = block_sum_int(c, red);
  if (threadIdx.x == 0) counts[e] = c;
}

// One workgroup of 1024 threads, thread e holding expert e (E <= 1024): an
// inclusive scan of (rows, tiles) within each wave, then across the waves.
__global__ __launch_bounds__(1024) void moe_scan_kernel(const int32_t* __restrict__ counts, int E,
                                                        int tile_rows, int32_t* __restrict__ seg_off,
                                                        int32_t* __restrict__ tile_off) {
  __shared__ int wr[16], wt[16];
  const int e = threadIdx.x, wave = e >> 6, lane = e & 63;
  const int c = e < E ? counts[e] : 0;
  const int tc = (c + tile_rows - 1) / tile_rows;
  int r = c, t = tc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ro = __shfl_up(r, o, 64), to = __shfl_up(t, o, 64);
    if (lane >= o) {
      r += ro;
      t += to;
    }
  }
  if (lane == 63) {
    wr[wave] = r;
    wt[wave] = t;
  }
  __syncthreads();
  int rb = 0, tb = 0;
  for (int w = 0; w < wave; ++w) {
    rb += wr[w];
    tb += wt[w];
  }
  r += rb;
  t += tb;
  if (e < E) {
    seg_off[e] = r - c;  // exclusive prefix
    tile_off[e] = t - tc;
  }
  if (e == E - 1) {
    seg_off[E] = r;
    tile_off[E] = t;
  }
}

__global__ __launch_bounds__(256) void moe_scatter_kernel(const int32_t* __restrict__ idx, int P,
                                                          int K, const int32_t* __restrict__ seg_off,
                                                          int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ inv) {
  __shared__ int wcount[4];
  const int e = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int base = seg_off[e];
  for (int i0 = 0; i0 < P; i0 += 256) {
    const int i = i0 + threadIdx.x;
    const bool hit = (i < P) && idx[i] == e;
    const uint64_t bal = __ballot(hit);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) wcount[wave] = __popcll(bal);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wcount[w];
    if (hit) {
      const int row = off + before;
      perm[row] = i / K;
      inv[i] = row;
    }
    base += wcount[0] + wcount[1] + wcount[2] + wcount[3];
  }
}

// One workgroup per token row; each thread covers 4 columns per pass.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ out,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ idx, int K,
                                                          int E, int D,
                                                          const float* __restrict__ shared_out,
                                                          uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 4; c < D; c += 256 * 4) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      if (e < 0 || e >= E) continue;
      const float wk = w[t * K + k];
      const f32x4 v = *reinterpret_cast<const f32x4*>(out + (size_t)inv[t * K + k] * D + c);
      a0 = __builtin_fmaf(wk, v[0], a0);
      a1 = __builtin_fmaf(wk, v[1], a1);
      a2 = __builtin_fmaf(wk, v[2], a2);
      a3 = __builtin_fmaf(wk, v[3], a3);
    }
    if (shared_out) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(shared_out + (size_t)t * D + c);
      a0 += v[0];
      a1 += v[1];
      a2 += v[2];
      a3 += v[3];
    }
    uint2 o;
    o.x = pack_bf2(a0, a1);
    o.y = pack_bf2(a2, a3);
    *reinterpret_cast<uint2*>(y + (size_t)t * D + c) = o;
  }
}

// z = bf16(o * sigmoid(g + b[head])) over [T][HD] with HD = Hq * hd; 8 per thread.
__global__ __launch_bounds__(256) void gate_kernel(const uint16_t* __restrict__ o,
                                                   const uint16_t* __restrict__ g,
                                                   const uint16_t* __restrict__ b, int hd, int HD,
                                                   long long n8, uint16_t* __restrict__ z) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 ov = ld16(o + i * 8), gv = ld16(g + i * 8);
  const float bb = bf2f(b[(int)((i * 8) % HD) / hd]);  // an 8-chunk never straddles heads
  const uint32_t* oi = reinterpret_cast<const uint32_t*>(&ov);
  const uint32_t* gi = reinterpret_cast<const uint32_t*>(&gv);
  uint32_t r[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    r[e] = pack_bf2(bf_lo(oi[e]) * sigmoidf_fast(bf_lo(gi[e]) + bb),
                    bf_hi(oi[e]) * sigmoidf_fast(bf_hi(gi[e]) + bb));
  *reinterpret_cast<uint4*>(z + i * 8) = uint4{r[0], r[1], r[2], r[3]};
}

int launch_moe_route(int T, int K, int E, const int32_t* idx, int tile_rows, int32_t* counts,
                     int32_t* seg_off, int32_t* tile_off, int32_t* perm, int32_t* inv,
                     hipStream_t st) {
  const int P = T * K;
  hipLaunchKernelGGL(moe_count_kernel, dim3(E), dim3(256), 0, st, idx, P, E, counts);
  if (E > 1024) return -1;
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(1024), 0, st, counts, E, tile_rows, seg_off,
                     tile_off);
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(E), dim3(256), 0, st, idx, P, K, seg_off, perm, inv);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_moe_combine(int T, int K, int E, int D, const float* out, const int32_t* inv,
                       const float* w, const int32_t* idx, const float* shared_out, uint16_t* y,
                       hipStream_t st) {
  hipLaunchKernelGGL(moe_combine_kernel, dim3(T), dim3(256), 0, st, out, inv, w, idx, K, E, D,
                     shared_out, y);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gate(int T, int Hq, int hd, const uint16_t* o, const uint16_t* g, const uint16_t* b,
                uint16_t* z, hipStream_t st) {
  const long long n8 = (long long)T * Hq * hd / 8;
  hipLaunchKernelGGL(gate_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, o, g, b,
                     hd, Hq * hd, n8, z);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace beam
