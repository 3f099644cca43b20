// bf16 matrix-core GEMMs for many-token (prefill) steps:
//   C[m][n] = sum_k A[m][k] * B[n][k]      A: activations [M][K], B: weight rows [N][K]
// fp32 accumulation on gfx950's v_mfma_f32_32x32x16_bf16.
//
// Tiling: a 256-thread workgroup owns a 256 x 256 tile of C; its 4 waves sit
// in a 2 x 2 grid and each owns 128 x 128 (4 x 4 MFMA blocks of 32 x 32,
// 256 fp32 accumulators per lane). K advances in slabs of 64: the next slab
// is loaded from global memory straight into the other half of a double
// buffer in LDS (no register staging) while the current one is multiplied
// out; inside a slab the operand fragments of k-step ks + 1 are read from LDS
// while the MFMAs of k-step ks run. LDS rows are 128 bytes (64 bf16), two to
// a 256-byte line of the 64 banks; the eight 16-byte chunks of row r are
// stored at chunk ^ ((r >> 1) & 7) so the 16-byte fragment reads of 16
// consecutive rows (16 lanes served per cycle) land on distinct banks.
//
// Variants (template Epi) cover the projections of the Beam layer ("Reflection
// Beam 1.0 on vLLM": packed q|k|v|gate GEMM of optimisation change 5, o_proj,
// the dense SwiGLU MLP of the MoE section, and the routed experts):
//   EPI_BF16   bf16 store, optionally split in two destinations at column n1
//   EPI_SWIGLU B rows are gate/up pairs; act = bf16(silu(bf16(g)) * bf16(u))
//   EPI_F32    fp32 store (per-(token, expert) rows for the weighted combine)
// Grouped mode: the M axis is a list of per-expert row segments; tile i maps to
// (expert, first row) through a prefix sum of per-expert tile counts, A rows
// may be gathered through an index list, and B is that expert's weight block.
//
// Tile order: workgroup b of the 1-D grid runs on XCD b % 8, and each XCD has
// its own L2. Each XCD therefore gets a contiguous eighth of the tile list,
// walked in column-major groups of kGroupM tile rows, so the ~32 tiles an XCD
// holds at once share a few A row panels and B column panels in its L2.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace beam {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGemmWaves = 8;  // waves per workgroup (4 or 8)
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

enum : int { EPI_BF16 = 0, EPI_SWIGLU = 1, EPI_F32 = 2 };

struct GemmArgs {
  int tiles_m, tiles_n;       // tile grid (tiles_m counts grouped-mode tile slots)
  const uint16_t* A;      // [M][lda] (or gathered rows)
  const uint16_t* B;      // [N][ldb] (per-expert base + e * b_expert_stride in grouped mode)
  int M, N, K;
  int lda, ldb;
  const int32_t* a_gather;    // row -> A row index (nullptr: identity)
  // grouped mode
  const int32_t* seg_off;     // [E+1] row offsets of the expert segments (nullptr: plain)
  const int32_t* tile_off;    // [E+1] prefix sums of per-expert M-tile counts
  int E;
  long long b_expert_stride;  // elements between experts' weight blocks
  const uint16_t* B_last;     // segment E - 1's weights when set (a shared expert)
  // epilogue
  void* out;
  int ldo;
  void* out2;                 // EPI_BF16 split destination (columns >= n1)
  int ldo2, n1;
  int F;                      // EPI_SWIGLU: up rows start at F (B row index)
  // split-K (EPI_F32 only): blockIdx.y = split z covers k-steps
  // [z * kt_split, (z + 1) * kt_split) and writes out + z * split_stride
  int kt_split;               // 0: the whole K range, no split
  long long split_stride;
};

// LDS slot of k-chunk `chunk` (16 B) in tile row `row` (BK = 64 bf16 = 128 B,
// two rows per 256-byte line of the 64 banks). A fragment read has 16 lanes
// in flight per cycle, on 16 consecutive rows: the 8 rows of one parity share
// a bank half, so they get 8 distinct slots from (row >> 1) & 7.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// WAVES = 4: waves in a 2 x 2 grid, 128 x 128 each (1 wave per SIMD);
// WAVES = 8: waves in a 2 x 4 grid, 128 x 64 each (2 waves per SIMD, so one
// issues MFMAs while the other waits on LDS).
// SKIP: MFMAs of 32-row blocks past the tile's last row are skipped (wave-
// uniform branches): for tiles expected to be mostly empty (grouped experts
// with few tokens each, or M well below the tile height).
// TR: tile rows (256, or 32 for grouped segments of a few rows each, which
// need only a 32-row A tile in LDS: 72 KiB instead of 128, two workgroups per
// CU, twice the weight streams in flight).
template <int EPI, int WAVES, bool SKIP, int TR = BM, int NS = 2>
__global__ __launch_bounds__(WAVES * 64) void gemm_bf16_kernel(GemmArgs g) {
  static_assert(TR == BM || (SKIP && TR == 32), "short tiles need the row skip");
  static_assert(NS == 2 || (NS == 4 && TR == 32), "a four-slab ring only for 32-row tiles");
  constexpr int WCOLS = WAVES / 2;     // wave grid columns
  constexpr int WN = BN / WCOLS;       // wave tile width (128 or 64)
  constexpr int TJ = WN / 32;          // 32-wide MFMA blocks per wave row
  constexpr int RPW = BM / WAVES;      // tile rows each wave loads (A and B)
  // K slabs in LDS (NS): two, or four for 32-row tiles bound by the weight
  // stream (three slabs in flight instead of one)
  extern __shared__ __align__(16) uint16_t lds[];
  // ring of NS slabs: A0 .. A(NS-1) | B0 .. B(NS-1)
  auto As = [&](int buf) { return lds + buf * (TR * BK); };
  auto Bs = [&](int buf) { return lds + NS * TR * BK + buf * (BN * BK); };

  // ---- workgroup -> tile (XCD-contiguous, grouped column-major) ---------------
  // Grouped mode launches the worst-case number of tile rows; only the first
  // tile_off[E] of them hold rows, so those are what gets split over the XCDs
  // (the rest of the grid exits at once instead of idling whole XCDs).
  // Grouped mode with full-height tiles walks the list expert by expert (an
  // expert's few tile rows, column-major): the ~32 tiles an XCD holds at once
  // then share one expert's A rows and read each of its B panels once, where
  // groups of kGroupM tile rows would span several experts and refetch their
  // A panels for every few columns.
  int tm, tn;
  {
    const int rows_m = g.seg_off ? g.tile_off[g.E] : g.tiles_m;
    const int nt = rows_m * g.tiles_n;
    const int b = blockIdx.x, x = b % kXcds, li = b / kXcds;
    const int q = nt / kXcds, r = nt % kXcds;
    if (li >= q + (x < r ? 1 : 0)) return;
    const int t = x * q + min(x, r) + li;  // this XCD's li-th tile
    if (TR == BM && g.seg_off) {
      int lo = 0, hi = g.E;  // largest e with tile_off[e] * tiles_n <= t (a non-empty expert)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (g.tile_off[mid] * g.tiles_n <= t) lo = mid; else hi = mid;
      }
      const int w = t - g.tile_off[lo] * g.tiles_n;
      const int rows = g.tile_off[lo + 1] - g.tile_off[lo];
      tm = g.tile_off[lo] + w % rows;
      tn = w / rows;
    } else {
      const int span = kGroupM * g.tiles_n;  // tiles per group of kGroupM tile rows
      const int grp = t / span, w = t - grp * span;
      const int rows = min(kGroupM, rows_m - grp * kGroupM);
      tm = grp * kGroupM + w % rows;
      tn = w / rows;
    }
  }
  // ---- tile -> (rows, expert) ------------------------------------------------
  int m0, mrows, e = 0;
  if (g.seg_off) {
    const int ti = tm;
    if (ti >= g.tile_off[g.E]) return;
    int lo = 0, hi = g.E;  // largest e with tile_off[e] <= ti
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g.tile_off[mid] <= ti) lo = mid; else hi = mid;
    }
    e = lo;
    const int seg0 = g.seg_off[e], seg1 = g.seg_off[e + 1];
    m0 = seg0 + (ti - g.tile_off[e]) * TR;
    mrows = min(TR, seg1 - m0);
  } else {
    m0 = tm * TR;
    mrows = min(TR, g.M - m0);
  }
  const int n0 = tn * BN;  // tile column origin (EPI_SWIGLU: in act columns x 2)
  const uint16_t* Bbase =
      (g.B_last && e == g.E - 1) ? g.B_last : g.B + (long long)e * g.b_expert_stride;

  // ---- global -> LDS loads ------------------------------------------------------
  // gfx950 loads 16 bytes per lane straight into LDS: one wave instruction
  // fills 1 KiB = 8 consecutive tile rows at a wave-uniform LDS address, lane l
  // landing at row l / 8, chunk slot l % 8. With the XOR swizzle, slot p of
  // row r holds k-chunk swz(r, p), so that is the chunk lane l fetches.
  // Wave w fills rows [RPW w, RPW (w + 1)) of the A and of the B tile.
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  constexpr int NL = RPW / 8;  // load instructions per wave and matrix
  const uint16_t* a_src[NL];
  const uint16_t* b_src[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int r = wave * RPW + i * 8 + (lane >> 3);
    const int c = swz(r, lane & 7);
    const int rr = min(r, mrows - 1);
    const int arow = g.a_gather ? g.a_gather[m0 + rr] : m0 + rr;
    a_src[i] = g.A + (long long)arow * g.lda + c * 8;
    int brow;
    if constexpr (EPI == EPI_SWIGLU) {
      // local column r: wave column wc = r / WN; within it WN/2 gate then WN/2 up
      const int wc = r / WN, cc = r % WN;
      const int f = (n0 >> 1) + wc * (WN / 2) + (cc % (WN / 2));
      brow = (cc < WN / 2) ? f : g.F + f;
      brow = min(brow, (cc < WN / 2 ? g.F : 2 * g.F) - 1);
    } else {
      brow = min(n0 + r, g.N - 1);
    }
    b_src[i] = Bbase + (long long)brow * g.ldb + c * 8;
  }
  auto gload = [&](int k0, int buf) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      // SKIP: A rows past the tile's last row are not fetched (their LDS rows
      // only feed outputs that are never stored); with 32-row tiles all of
      // wave 0's A rows are (clamped to the last row), so every wave issues a
      // fixed number of copies per slab
      if (!SKIP || wave * RPW + i * 8 < (NS > 2 ? TR : mrows))  // (mrows <= TR)
        load_lds16(a_src[i] + k0, As(buf) + (wave * RPW + i * 8) * BK);
      load_lds16(b_src[i] + k0, Bs(buf) + (wave * RPW + i * 8) * BK);
    }
  };

  const int wm = wave / WCOLS, wn = wave % WCOLS;
  const int band = mrows - wm * 128;  // rows of this wave's 128-row band that exist
  const int lr = lane & 31, lk = lane >> 5;  // fragment row / k half
  // 32-row blocks a wave can own: 4, or 1 with 32-row tiles (then only the
  // first wave row holds rows at all; the accumulators shrink to fit two
  // workgroups per CU)
  constexpr int MI = TR >= 128 ? 4 : 1;
  f32x16 acc[MI][TJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

  // fragments of k-step ks (16 deep) of buffer buf
  auto frags = [&](int buf, int ks, bf16x8 (&af)[MI], bf16x8 (&bfr)[TJ]) {
    const uint16_t* Ab = As(buf) + (wm * 128) * BK;
    const uint16_t* Bb = Bs(buf) + (wn * WN) * BK;
    const int chunk = ks * 2 + lk;  // 8 bf16 = one 16 B chunk
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = i * 32 + lr;
      af[i] = *reinterpret_cast<const bf16x8*>(Ab + r * BK + swz(r, chunk) * 8);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int r = j * 32 + lr;
      bfr[j] = *reinterpret_cast<const bf16x8*>(Bb + r * BK + swz(r, chunk) * 8);
    }
  };

  const int kt0 = g.kt_split ? blockIdx.y * g.kt_split : 0;
  const int KT = g.kt_split ? kt0 + g.kt_split : g.K / BK;
  // Ring: this wave's copies of one slab are NL (B rows) plus, in wave 0 of a
  // 32-row tile, NL more (A rows). Waiting for slab kt + 1 leaves the copies
  // of the `ahead` slabs issued after it in flight; the barrier then makes
  // every wave's copies of slab kt + 1 visible, and no wave still reads the
  // slab the next copy overwrites (its fragment reads have completed).
  const int per_slab = (NS > 2 && wave == 0) ? 2 * NL : NL;
  auto ring_barrier = [&](int ahead) {
    const int n = ahead * per_slab;  // 0, NL, 2 NL or 4 NL
    if (n == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if (n == NL) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NL) : "memory");
    else if (n == 2 * NL)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * NL) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(4 * NL) : "memory");
  };
  if constexpr (NS == 2) {
    gload(kt0 * BK, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  } else {
    const int pre = min(NS - 1, KT - kt0);  // slabs requested ahead of the loop
    for (int p = 0; p < pre; ++p) gload((kt0 + p) * BK, p);
    ring_barrier(max(0, pre - 1));
  }
  // Two copies of the K loop: one with the per-block row skip, one without its
  // branches. A wave whose row blocks all hold rows takes the branch-free copy,
  // so SKIP costs full tiles nothing (both copies meet the same barriers).
  auto kloop = [&](auto skip_tag) {
    constexpr bool SK = decltype(skip_tag)::value;
    for (int kt = kt0; kt < KT; ++kt) {
      const int cur = (kt - kt0) % NS;  // slot 0 holds the first k-step of this split
      // the slot copied into was last read in step kt - 1, which every wave has left
      if (kt + NS - 1 < KT) gload((kt + NS - 1) * BK, (kt - kt0 + NS - 1) % NS);
      bf16x8 af[2][MI], bfr[2][TJ];
      frags(cur, 0, af[0], bfr[0]);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        if (ks + 1 < BK / 16) frags(cur, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if (SK && 32 * i >= band) continue;
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j],
                                                               acc[i][j], 0, 0, 0);
        }
      }
      if constexpr (NS == 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of step kt + 1
        __syncthreads();
      } else {
        ring_barrier(max(0, min(NS - 2, KT - 2 - kt)));  // slabs kt + 2 .. issued
      }
    }
  };
  if (SKIP && band < MI * 32) kloop(std::integral_constant<bool, SKIP>{});
  else kloop(std::integral_constant<bool, false>{});

  // ---- epilogue -------------------------------------------------------------------
  // acc[i][j][4*ii + jj] = C[row 32 i + 8 ii + 4 lk + jj][col 32 j + lr] of the wave tile
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int rloc = wm * 128 + 32 * i + 8 * ii + 4 * lk + jj;
        if (rloc >= mrows) continue;
        const long long m = m0 + rloc;
        if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
          for (int j = 0; j < TJ / 2; ++j) {
            const int f = (n0 >> 1) + wn * (WN / 2) + 32 * j + lr;
            if (f < g.F) {
              const float gt = round_bf(acc[i][j][4 * ii + jj]);
              const float up = round_bf(acc[i][j + TJ / 2][4 * ii + jj]);
              reinterpret_cast<uint16_t*>(g.out)[m * g.ldo + f] = f2bf(siluf(gt) * up);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const int n = n0 + wn * WN + 32 * j + lr;
            if (n >= g.N) continue;
            const float v = acc[i][j][4 * ii + jj];
            if constexpr (EPI == EPI_F32) {
              reinterpret_cast<float*>(g.out)[blockIdx.y * g.split_stride + m * g.ldo + n] = v;
            } else {
              if (n < g.n1)
                reinterpret_cast<uint16_t*>(g.out)[m * g.ldo + n] = f2bf(v);
              else
                reinterpret_cast<uint16_t*>(g.out2)[m * g.ldo2 + (n - g.n1)] = f2bf(v);
            }
          }
        }
      }
    }
  }
}

static size_t gemm_lds_bytes(int tr = BM, int ns = 2) { return (size_t)ns * (tr + BN) * BK * 2; }

template <int EPI, bool SKIP = false, int TR = BM, int WAVES = kGemmWaves, int NS = 2>
static int launch(const GemmArgs& a, int grid_n, int grid_m, hipStream_t st, int splits = 1) {
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_bf16_kernel<EPI, WAVES, SKIP, TR, NS>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)gemm_lds_bytes(TR, NS));
    attr_set = true;
  }
  GemmArgs g = a;
  g.tiles_m = grid_m;
  g.tiles_n = grid_n;
  hipLaunchKernelGGL((gemm_bf16_kernel<EPI, WAVES, SKIP, TR, NS>), dim3(grid_m * grid_n, splits),
                     dim3(WAVES * 64), gemm_lds_bytes(TR, NS), st, g);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------------------------
// Split-K for short, wide products (a batch of decode steps: M <= 256 tokens
// against a weight whose N / 256 column tiles alone would leave most of the
// chip idle). Each split multiplies a slice of K into an fp32 partial
// [split][M][N]; gemm_split_reduce adds the partials in split order and
// applies the epilogue (bf16 store with optional column split, or SwiGLU of
// the gate / up column halves).
// Tile rows of the split product: 32-row tiles for at most 128 tokens (72 KiB
// of LDS, two workgroups per CU, so twice the splits are in flight), else 256.
static int split_rows(int M) { return M <= 128 ? 32 : BM; }

int gemm_splits(int M, int N, int K) {
  if (M > BM || K % BK) return 1;
  const int tr = split_rows(M);
  const int tiles = ((M + tr - 1) / tr) * ((N + BN - 1) / BN);
  const int cap = tr == BM ? 256 : 512;  // workgroups the chip holds at once
  const int ks = K / BK;
  int s = 1;
  // the partials (written, then read back) stay within half the weight bytes
  while (tiles * s * 2 <= cap && ks % (s * 2) == 0 && (long long)s * 2 * 4 * M <= K) s *= 2;
  return s;
}

size_t gemm_split_bytes(int M, int N, int K) {
  const int s = gemm_splits(M, N, K);
  return s > 1 ? (size_t)s * M * N * 4 : 0;
}

// EPI_BF16: out[m][n] (n < n1) or out2[m][n - n1]; EPI_SWIGLU: out[m][f] =
// bf16(silu(bf16(g)) * bf16(u)) with g, u the partial sums of columns f, F + f.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(
    const float* __restrict__ part, int splits, int M, int N, uint16_t* __restrict__ out,
    int ldo, uint16_t* __restrict__ out2, int ldo2, int n1, int F) {
  const int ncols = EPI == EPI_SWIGLU ? F : N;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)M * ncols) return;
  const int m = (int)(i / ncols), n = (int)(i - (long long)m * ncols);
  const size_t ss = (size_t)M * N;
  if constexpr (EPI == EPI_SWIGLU) {
    float gt = 0.f, up = 0.f;
    for (int z = 0; z < splits; ++z) {
      gt += part[z * ss + (size_t)m * N + n];
      up += part[z * ss + (size_t)m * N + F + n];
    }
    out[(size_t)m * ldo + n] = f2bf(siluf(round_bf(gt)) * round_bf(up));
  } else {
    float v = 0.f;
    for (int z = 0; z < splits; ++z) v += part[z * ss + (size_t)m * N + n];
    if (n < n1) out[(size_t)m * ldo + n] = f2bf(v);
    else out2[(size_t)m * ldo2 + (n - n1)] = f2bf(v);
  }
}

template <int EPI>
static int launch_split(const GemmArgs& a0, int splits, float* part, hipStream_t st) {
  GemmArgs a = a0;
  a.out = part;
  a.ldo = a.N;
  a.kt_split = a.K / BK / splits;
  a.split_stride = (long long)a.M * a.N;
  const int tr = split_rows(a.M);
  const int tn = (a.N + BN - 1) / BN, tm = (a.M + tr - 1) / tr;
  if (tr == BM ? launch<EPI_F32, true>(a, tn, tm, st, splits)
               : launch<EPI_F32, true, 32>(a, tn, tm, st, splits))
    return -1;
  const long long n = (long long)a.M * (EPI == EPI_SWIGLU ? a0.F : a.N);
  hipLaunchKernelGGL((gemm_split_reduce_kernel<EPI>), dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, st, part, splits, a.M, a.N,
                     reinterpret_cast<uint16_t*>(a0.out), a0.ldo,
                     reinterpret_cast<uint16_t*>(a0.out2), a0.ldo2, a0.n1, a0.F);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gemm_bf16(int M, int N, int K, const uint16_t* A, int lda, const uint16_t* B, int ldb,
                     uint16_t* out, int ldo, uint16_t* out2, int ldo2, int n1, float* part,
                     hipStream_t st) {
  GemmArgs a{};
  a.A = A; a.B = B; a.M = M; a.N = N; a.K = K; a.lda = lda; a.ldb = ldb;
  a.out = out; a.ldo = ldo; a.out2 = out2; a.ldo2 = ldo2; a.n1 = out2 ? n1 : N;
  const int s = gemm_splits(M, N, K);
  if (s > 1 && part) return launch_split<EPI_BF16>(a, s, part, st);
  if (M <= BM / 2) return launch<EPI_BF16, true>(a, (N + BN - 1) / BN, (M + BM - 1) / BM, st);
  return launch<EPI_BF16>(a, (N + BN - 1) / BN, (M + BM - 1) / BM, st);
}

int launch_gemm_swiglu(int M, int F, int K, const uint16_t* A, int lda, const int32_t* gather,
                       const uint16_t* B, const int32_t* seg_off, const int32_t* tile_off, int E,
                       long long b_stride, int max_mtiles, uint16_t* act, float* part,
                       hipStream_t st, const uint16_t* B_last) {
  GemmArgs a{};
  a.A = A; a.B = B; a.M = M; a.N = 2 * F; a.K = K; a.lda = lda; a.ldb = K;
  a.a_gather = gather; a.seg_off = seg_off; a.tile_off = tile_off; a.E = E;
  a.B_last = seg_off ? B_last : nullptr;
  a.b_expert_stride = b_stride; a.out = act; a.ldo = F; a.F = F; a.n1 = 2 * F;
  if (!seg_off) {
    const int s = gemm_splits(M, 2 * F, K);
    if (s > 1 && part) return launch_split<EPI_SWIGLU>(a, s, part, st);
  }
  const int gn = (2 * F + BN - 1) / BN;
  // the gate/up rows (K = D) stream through a four-slab ring: one workgroup
  // per CU with three slabs in flight beats two with one each here
  if (seg_off && gemm_grouped_rows(M, E) == 32)
    return launch<EPI_SWIGLU, true, 32, kGemmWaves, 4>(a, gn, max_mtiles, st);
  const int gm = seg_off ? max_mtiles : (M + BM - 1) / BM;
  if (seg_off || M <= BM / 2) return launch<EPI_SWIGLU, true>(a, gn, gm, st);
  return launch<EPI_SWIGLU>(a, gn, gm, st);
}

int launch_gemm_f32(int M, int N, int K, const uint16_t* A, int lda, const uint16_t* B,
                    const int32_t* seg_off, const int32_t* tile_off, int E, long long b_stride,
                    int max_mtiles, float* out, int ldo, hipStream_t st, const uint16_t* B_last) {
  GemmArgs a{};
  a.A = A; a.B = B; a.M = M; a.N = N; a.K = K; a.lda = lda; a.ldb = K;
  a.seg_off = seg_off; a.tile_off = tile_off; a.E = E; a.b_expert_stride = b_stride;
  a.B_last = seg_off ? B_last : nullptr;
  a.out = out; a.ldo = ldo; a.n1 = N;
  const int gn = (N + BN - 1) / BN;
  if (seg_off && gemm_grouped_rows(M, E) == 32)
    return launch<EPI_F32, true, 32>(a, gn, max_mtiles, st);
  const int gm = seg_off ? max_mtiles : (M + BM - 1) / BM;
  if (seg_off || M <= BM / 2) return launch<EPI_F32, true>(a, gn, gm, st);
  return launch<EPI_F32>(a, gn, gm, st);
}

// Tile rows of the grouped expert GEMMs for M (token, slot) rows over E
// experts: 32 when the segments average at most 16 rows (a batch of decode
// steps), else 256. The routing permutation is built with the same value.
int gemm_grouped_rows(int M, int E) { return (long long)M <= 16LL * E ? 32 : BM; }

}  // namespace beam
