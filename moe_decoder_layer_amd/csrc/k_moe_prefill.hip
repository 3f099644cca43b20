// Many-token expert dispatch for the routed SwiGLU experts ("Reflection Beam
// 1.0 on vLLM", MoE section: every token goes to its 8 selected experts; the
// page's decode graph uses two routing kernels and two grouped GEMMs).
//
//   moe_count_kernel    per chunk of pairs, the count of each expert
//   moe_scan_kernel     row offsets of the expert segments, prefix sums of
//                       their GEMM tile counts, each chunk's base per expert
//   moe_scatter_kernel  one workgroup per chunk writes its pairs in (token,
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

// The (token, slot) pairs are cut into chunks of moe_route_chunk(P) pairs (a
// multiple of 256); chunk c's per-expert counts go to counts[c][E].
// Expert of pair i of the (token, slot) list, spt slots per token: slots
// 0..K-1 hold the routed experts of idx (-1 for an id outside [0, E)), slot K
// (when spt = K + 1) the shared expert, numbered E.
__device__ __forceinline__ int pair_expert(const int32_t* __restrict__ idx, int i, int K, int spt,
                                           int E) {
  const int t = i / spt, s = i - t * spt;
  if (s >= K) return E;
  const int v = idx[t * K + s];
  return (v >= 0 && v < E) ? v : -1;
}

// NE segments: the E routed experts, plus the shared expert when spt > K.
__global__ __launch_bounds__(256) void moe_count_kernel(const int32_t* __restrict__ idx, int P,
                                                        int K, int spt, int E, int NE,
                                                        int chunk,
                                                        int32_t* __restrict__ counts) {
  __shared__ int hist[1024];
  const int c = blockIdx.x, i0 = c * chunk, i1 = min(P, i0 + chunk);
  for (int e = threadIdx.x; e < NE; e += 256) hist[e] = 0;
  __syncthreads();
  for (int i = i0 + threadIdx.x; i < i1; i += 256) {
    const int v = pair_expert(idx, i, K, spt, E);
    if (v >= 0) atomicAdd(&hist[v], 1);  // an integer count: order-independent
    else BEAM_RAISE(moe, ERR_EXPERT);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < NE; e += 256) counts[(size_t)c * NE + e] = hist[e];
}

// One workgroup of 1024 threads, thread e holding expert e (E <= 1024): its
// total over the chunks, an inclusive scan of (rows, tiles) over the experts
// (within each wave, then across the waves), and then counts[c][e] replaced
// by the row where chunk c's first pair of expert e goes.
__global__ __launch_bounds__(1024) void moe_scan_kernel(int32_t* __restrict__ counts, int nch,
                                                        int E, int tile_rows,
                                                        int32_t* __restrict__ seg_off,
                                                        int32_t* __restrict__ tile_off) {
  __shared__ int wr[16], wt[16];
  const int e = threadIdx.x, wave = e >> 6, lane = e & 63;
  int c = 0;
  if (e < E)
    for (int ch = 0; ch < nch; ++ch) c += counts[(size_t)ch * E + e];
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
    int run = r - c;
    for (int ch = 0; ch < nch; ++ch) {
      const int n = counts[(size_t)ch * E + e];
      counts[(size_t)ch * E + e] = run;
      run += n;
    }
  }
  if (e == E - 1) {
    seg_off[E] = r;
    tile_off[E] = t;
  }
}

// One workgroup per chunk, its pairs in order, 256 at a time: a pair's row is
// its expert's running base for the chunk plus the number of earlier pairs of
// the same expert in the batch of 256 (pairs keep (token, slot) order within
// every expert). perm[row] = token, inv[pair] = row.
__global__ __launch_bounds__(256) void moe_scatter_kernel(const int32_t* __restrict__ idx, int P,
                                                          int K, int spt, int E, int NE,
                                                          int chunk,
                                                          const int32_t* __restrict__ base,
                                                          int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ inv) {
  __shared__ int run[1024];
  __shared__ int ex[256];
  const int c = blockIdx.x, i0 = c * chunk, i1 = min(P, i0 + chunk);
  for (int e = threadIdx.x; e < NE; e += 256) run[e] = base[(size_t)c * NE + e];
  for (int b0 = i0; b0 < i1; b0 += 256) {
    const int i = b0 + threadIdx.x;
    const int v = i < i1 ? pair_expert(idx, i, K, spt, E) : -1;
    const bool ok = v >= 0;
    __syncthreads();  // run[] updated by the previous batch
    ex[threadIdx.x] = ok ? v : -1;
    __syncthreads();
    int before = 0;
    if (ok)
      for (int j = 0; j < (int)threadIdx.x; ++j) before += (ex[j] == v);
    const int row = ok ? run[v] + before : 0;
    __syncthreads();  // every lane has read run[] for this batch
    if (ok) {
      perm[row] = i / spt;
      inv[i] = row;
      atomicAdd(&run[v], 1);  // an integer count: order-independent
    }
  }
}

// The whole routing in one workgroup for at most 2,048 pairs (a batch of
// decode steps), with the same results as the three kernels above: per-expert
// counts by LDS atomics, the scan of (rows, tiles), then the pairs ranked in
// (token, slot) order, 1,024 at a time. Within a wave, the lanes that share an
// expert are found one distinct expert per round (a ballot against the first
// unresolved lane's expert); each wave's lowest lane per expert enters the
// group's size in a [wave][expert] table, and thread e turns expert e's column
// into each wave's first row (a prefix over the waves in order).
constexpr int kRouteSmallMax = 2048;

__global__ __launch_bounds__(1024) void moe_route_small_kernel(
    const int32_t* __restrict__ idx, int P, int K, int spt, int E, int NE, int tile_rows,
    int32_t* __restrict__ seg_off, int32_t* __restrict__ tile_off, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv) {
  __shared__ int run[1024];
  __shared__ int wcnt[16 * 1024];
  __shared__ int wr[16], wt[16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int ev[2];  // experts of pairs tid and tid + 1024 (-1: an id outside [0, E); -2: no pair)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = tid + h * 1024;
    ev[h] = i < P ? pair_expert(idx, i, K, spt, E) : -2;
    if (ev[h] == -1) BEAM_RAISE(moe, ERR_EXPERT);
  }
  if (tid < NE) run[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (ev[h] >= 0) atomicAdd(&run[ev[h]], 1);  // an integer count: order-independent
  __syncthreads();
  // thread e: expert e's rows and tiles, inclusive scan within the wave, then
  // across the waves
  const int c = tid < NE ? run[tid] : 0;
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
  for (int w = 0; w < wave; ++w) {
    r += wr[w];
    t += wt[w];
  }
  if (tid < NE) {
    seg_off[tid] = r - c;  // exclusive prefix
    tile_off[tid] = t - tc;
    run[tid] = r - c;      // the next row of expert tid
  }
  if (tid == NE - 1) {
    seg_off[NE] = r;
    tile_off[NE] = t;
  }
  __syncthreads();
  for (int h = 0; h < 2 && h * 1024 < P; ++h) {
    const int i = tid + h * 1024, v = ev[h];
    const bool ok = v >= 0;
    uint64_t same = 0;  // lanes of this wave with expert v
    uint64_t pend = __ballot(ok);
    while (pend) {
      const int lead = __ffsll((unsigned long long)pend) - 1;
      const int lv = __shfl(v, lead, 64);
      const uint64_t m = __ballot(ok && v == lv);
      if (ok && v == lv) same = m;
      pend &= ~m;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1));
    // wcnt[w][e]: pairs of expert e in wave w, then wave w's first row for e
    // (cleared once every wave has read its rows of the previous batch)
    __syncthreads();
    for (int k = tid; k < 16 * NE; k += 1024) wcnt[k] = 0;
    __syncthreads();
    if (ok && rank == 0) wcnt[wave * NE + v] = __popcll(same);
    __syncthreads();
    if (tid < NE) {
      int row = run[tid];
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const int n = wcnt[w * NE + tid];
        wcnt[w * NE + tid] = row;
        row += n;
      }
      run[tid] = row;
    }
    __syncthreads();
    if (ok) {
      const int row = wcnt[wave * NE + v] + rank;
      perm[row] = i / spt;
      inv[i] = row;
    }
  }
}

// One workgroup per token row; each thread covers 4 columns per pass.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ out,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ idx, int K,
                                                          int spt, int E, int D,
                                                          uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 4; c < D; c += 256 * 4) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      if (e < 0 || e >= E) continue;
      const float wk = w[t * K + k];
      const f32x4 v = *reinterpret_cast<const f32x4*>(out + (size_t)inv[t * spt + k] * D + c);
      a0 = __builtin_fmaf(wk, v[0], a0);
      a1 = __builtin_fmaf(wk, v[1], a1);
      a2 = __builtin_fmaf(wk, v[2], a2);
      a3 = __builtin_fmaf(wk, v[3], a3);
    }
    if (spt > K) {  // the shared expert's row, weight 1
      const f32x4 v = *reinterpret_cast<const f32x4*>(out + (size_t)inv[t * spt + K] * D + c);
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

// The same combine for at most KM routed slots: the token's ids, weights and
// rows are requested once, before any row, and each pass requests every slot's
// row chunk before the first product (the products and sums in the order of
// moe_combine_kernel, so both give identical results).
template <int KM>
__global__ __launch_bounds__(256) void moe_combine_rows_kernel(const float* __restrict__ out,
                                                               const int32_t* __restrict__ inv,
                                                               const float* __restrict__ w,
                                                               const int32_t* __restrict__ idx,
                                                               int K, int spt, int E, int D,
                                                               uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  const bool shared = spt > K;
  bool ok[KM];
  float wk[KM];
  size_t row[KM + 1];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int e = k < K ? idx[t * K + k] : -1;
    ok[k] = e >= 0 && e < E;  // an id outside [0, E): its slot has no row
    wk[k] = ok[k] ? w[t * K + k] : 0.f;
    row[k] = ok[k] ? (size_t)inv[t * spt + k] * D : 0;
  }
  row[KM] = shared ? (size_t)inv[t * spt + K] * D : 0;
  for (int c = threadIdx.x * 4; c < D; c += 256 * 4) {
    f32x4 v[KM + 1];
#pragma unroll
    for (int k = 0; k < KM; ++k)
      v[k] = ok[k] ? *reinterpret_cast<const f32x4*>(out + row[k] + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    v[KM] = shared ? *reinterpret_cast<const f32x4*>(out + row[KM] + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (!ok[k]) continue;
      a0 = __builtin_fmaf(wk[k], v[k][0], a0);
      a1 = __builtin_fmaf(wk[k], v[k][1], a1);
      a2 = __builtin_fmaf(wk[k], v[k][2], a2);
      a3 = __builtin_fmaf(wk[k], v[k][3], a3);
    }
    if (shared) {  // the shared expert's row, weight 1
      a0 += v[KM][0];
      a1 += v[KM][1];
      a2 += v[KM][2];
      a3 += v[KM][3];
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

// Pairs per routing chunk: 256 for short spans (a batch of decode steps), so
// the scatter's per-batch ranking runs in several workgroups at once, doubled
// up to 2048 while there would be more than 64 chunks, so the scan's walk over
// the chunks stays short.
static int moe_route_chunk(int P) {
  int c = 256;
  while (c < 2048 && (P + c - 1) / c > 64) c *= 2;
  return c;
}

int moe_route_chunks(int P) {
  const int c = moe_route_chunk(P);
  return (P + c - 1) / c;
}

int launch_moe_route(int T, int K, int spt, int E, const int32_t* idx, int tile_rows,
                     int32_t* counts, int32_t* seg_off, int32_t* tile_off, int32_t* perm,
                     int32_t* inv, hipStream_t st) {
  const int P = T * spt, NE = E + (spt > K ? 1 : 0);
  if (NE > 1024) return -1;
  if (P <= kRouteSmallMax) {
    hipLaunchKernelGGL(moe_route_small_kernel, dim3(1), dim3(1024), 0, st, idx, P, K, spt, E, NE,
                       tile_rows, seg_off, tile_off, perm, inv);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int chunk = moe_route_chunk(P), nch = moe_route_chunks(P);
  hipLaunchKernelGGL(moe_count_kernel, dim3(nch), dim3(256), 0, st, idx, P, K, spt, E, NE, chunk,
                     counts);
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(1024), 0, st, counts, nch, NE, tile_rows,
                     seg_off, tile_off);
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(nch), dim3(256), 0, st, idx, P, K, spt, E, NE,
                     chunk, counts, perm, inv);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_moe_combine(int T, int K, int spt, int E, int D, const float* out, const int32_t* inv,
                       const float* w, const int32_t* idx, uint16_t* y, hipStream_t st) {
  if (K <= 8)
    hipLaunchKernelGGL((moe_combine_rows_kernel<8>), dim3(T), dim3(256), 0, st, out, inv, w, idx,
                       K, spt, E, D, y);
  else
    hipLaunchKernelGGL(moe_combine_kernel, dim3(T), dim3(256), 0, st, out, inv, w, idx, K, spt, E,
                       D, y);
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
