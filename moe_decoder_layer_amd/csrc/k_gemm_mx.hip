// Grouped expert GEMMs on block-scaled operands for many-token steps: the
// routed experts of the MoE section ("Reflection Beam 1.0 on vLLM" runs them
// in a 4-bit block format; the optimisation section's library MoE path
// quantises the activations for it and runs two grouped GEMMs). Here the
// activations are MXFP8 (e4m3 codes, one E8M0 scale per 32 along K, the
// weights' rule) and the expert weights MXFP8 or MXFP4 (e2m1 codes, two per
// byte), multiplied on gfx950's scaled matrix cores:
//   C[m][n] = sum_k decode(A[m][k]) 2^(sA[m][k/32] - 127) decode(B[n][k]) 2^(sB[n][k/32] - 127)
// with v_mfma_scale_f32_32x32x64_f8f6f4 (fp32 accumulation).
//
// Operand layout of that instruction (measured): lane (r, h) = (lane % 32,
// lane / 32) supplies row r (A) or column r (B) and the scale of K-block h of
// the 64-deep step; an e4m3 operand holds k in 16 h + [0, 16) in its first 16
// bytes and 32 + 16 h + [0, 16) in the next 16, an e2m1 operand k in 32 h +
// [0, 32) in 16 bytes.
//
// Tiling as the bf16 grouped GEMM: a 512-thread workgroup owns a 256 x 256
// tile of one expert's rows, its 8 waves in a 2 x 4 grid (128 x 64 each);
// K advances in slabs of 128 loaded from global memory straight into a
// double-buffered LDS tile (16 bytes per lane), the next slab in flight while
// the current one is multiplied out. A rows and e4m3 B rows are 128 bytes per
// slab (16-byte chunk c of row r at slot c ^ ((r >> 1) & 7)), e2m1 B rows 64
// bytes (slot c ^ ((r >> 2) & 3)): the 16-byte reads of 16 consecutive rows
// hit 16 distinct slots of the 64 banks. The scale words (four K-blocks of a
// row per slab in one 32-bit word) travel with the slabs: each wave loads the
// words of 64 A or B rows straight into LDS, so every row's words are fetched
// once per workgroup, and the lanes read theirs from LDS. When K is a multiple
// of 512 a row's 16 bytes of four consecutive slabs come in one load, with
// the first of those slabs; otherwise each slab brings its own word.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace beam {

namespace {

constexpr int XBM = 256, XBN = 256, XBK = 128;  // tile rows, columns, slab depth
constexpr int XWAVES = 8;
constexpr int kXcdsMx = 8;

typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int sw8(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ int sw4(int r, int c) { return c ^ ((r >> 2) & 3); }

struct MxGemmArgs {
  const uint8_t* A;         // activation codes [rows][K] (e4m3)
  const uint8_t* As;        // their scales [rows][K / 32]
  const int32_t* a_gather;  // C row -> A row (nullptr: identity)
  const uint8_t* B;         // expert 0's weight codes [N][K] (e4m3) or [N][K / 2] (e2m1)
  const uint8_t* Bs;        // expert 0's scales [N][K / 32]
  long long b_stride, bs_stride;  // bytes between consecutive experts
  int N, K;
  const int32_t* seg_off;   // [E + 1] row offsets of the expert segments
  const int32_t* tile_off;  // [E + 1] prefix sums of per-expert tile counts
  int E;
  int tiles_n;
  void* out;                // SwiGLU: act [rows][F] bf16; else fp32 [rows][ldo]
  int ldo, F;
};

}  // namespace

enum : int { MX_EPI_SWIGLU = 1, MX_EPI_F32 = 2 };

template <int EPI, bool B4>
__global__ __launch_bounds__(XWAVES * 64) void gemm_mx_kernel(MxGemmArgs g) {
  constexpr int BROW = B4 ? XBK / 2 : XBK;  // bytes of a B row per slab
  constexpr int WCOLS = XWAVES / 2, WN = XBN / WCOLS, TJ = WN / 32, MI = 4;
  constexpr int RPW = XBM / XWAVES;           // rows each wave loads (32)
  extern __shared__ __align__(16) uint8_t lds8[];
  auto Asl = [&](int buf) { return lds8 + buf * (XBM * XBK); };
  auto Bsl = [&](int buf) { return lds8 + 2 * XBM * XBK + buf * (XBN * BROW); };
  // scale words, A rows [0, 256) then B rows [256, 512): per buffer the four
  // slabs of a group ([row][4] words, g4) or one slab ([row] words)
  auto Ssl = [&](int buf) {
    return reinterpret_cast<uint32_t*>(lds8 + 2 * XBM * XBK + 2 * XBN * BROW) +
           buf * 4 * (XBM + XBN);
  };

  // ---- workgroup -> tile: XCD-contiguous, expert by expert ---------------------
  int tm, tn;
  {
    const int rows_m = g.tile_off[g.E];
    const int nt = rows_m * g.tiles_n;
    const int b = blockIdx.x, x = b % kXcdsMx, li = b / kXcdsMx;
    const int q = nt / kXcdsMx, r = nt % kXcdsMx;
    if (li >= q + (x < r ? 1 : 0)) return;
    const int t = x * q + min(x, r) + li;
    int lo = 0, hi = g.E;  // largest e with tile_off[e] * tiles_n <= t (a non-empty expert)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g.tile_off[mid] * g.tiles_n <= t) lo = mid; else hi = mid;
    }
    const int w = t - g.tile_off[lo] * g.tiles_n;
    const int rows = g.tile_off[lo + 1] - g.tile_off[lo];
    tm = g.tile_off[lo] + w % rows;
    tn = w / rows;
  }
  int e;
  {
    int lo = 0, hi = g.E;  // largest e with tile_off[e] <= tm
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g.tile_off[mid] <= tm) lo = mid; else hi = mid;
    }
    e = lo;
  }
  const int m0 = g.seg_off[e] + (tm - g.tile_off[e]) * XBM;
  const int mrows = min(XBM, g.seg_off[e + 1] - m0);
  const int n0 = tn * XBN;
  const uint8_t* Bc = g.B + (long long)e * g.b_stride;
  const uint8_t* Bsc = g.Bs + (long long)e * g.bs_stride;
  const int K = g.K, ksc = K / 32;  // scale bytes per row

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // B row of local tile column r (SwiGLU: the wave columns hold WN / 2 gate
  // then WN / 2 up rows)
  auto brow_of = [&](int r) {
    if constexpr (EPI == MX_EPI_SWIGLU) {
      const int wc = r / WN, cc = r % WN;
      const int f = (n0 >> 1) + wc * (WN / 2) + (cc % (WN / 2));
      const int br = (cc < WN / 2) ? f : g.F + f;
      return min(br, (cc < WN / 2 ? g.F : 2 * g.F) - 1);
    } else {
      return min(n0 + r, g.N - 1);
    }
  };
  auto arow_of = [&](int r) {
    const int rr = min(r, mrows - 1);
    return g.a_gather ? g.a_gather[m0 + rr] : m0 + rr;
  };

  // ---- global -> LDS: one wave instruction fills 1 KiB ------------------------
  // A and e4m3 B: 8 rows of 8 chunks, lane l at row l / 8, slot l % 8 (holding
  // chunk sw8(row, l % 8)); e2m1 B: 16 rows of 4 chunks, lane l at row l / 4.
  constexpr int NA = RPW / 8, NB = B4 ? RPW / 16 : RPW / 8;
  uint32_t a_off[NA], b_off[NB];  // byte offsets at k = 0 (< 2^32: rows x K bytes)
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = wave * RPW + i * 8 + (lane >> 3);
    a_off[i] = (uint32_t)arow_of(r) * (uint32_t)K + (uint32_t)(sw8(r, lane & 7) * 16);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if constexpr (B4) {
      const int r = wave * RPW + i * 16 + (lane >> 2);
      b_off[i] = (uint32_t)brow_of(r) * (uint32_t)(K / 2) + (uint32_t)(sw4(r, lane & 3) * 16);
    } else {
      const int r = wave * RPW + i * 8 + (lane >> 3);
      b_off[i] = (uint32_t)brow_of(r) * (uint32_t)K + (uint32_t)(sw8(r, lane & 7) * 16);
    }
  }
  // scale words: wave w < 4 loads those of A rows 64 w + lane, wave w >= 4
  // those of B rows 64 (w - 4) + lane (row offsets in bytes, < 2^32)
  const uint8_t* s_src;
  uint32_t s_off;
  if (wave < 4) {
    s_src = g.As;
    s_off = (uint32_t)arow_of(64 * wave + lane) * (uint32_t)ksc;
  } else {
    s_src = Bsc;
    s_off = (uint32_t)brow_of(64 * (wave - 4) + lane) * (uint32_t)ksc;
  }
  const bool g4 = (ksc & 15) == 0;
  auto gload = [&](int kt, int buf) {
    if (!g4)
      load_lds4(s_src + s_off + (uint32_t)kt * 4, Ssl(buf) + 64 * wave);
    else if ((kt & 3) == 0)  // this group's buffer was last read four slabs ago
      load_lds16(s_src + s_off + (uint32_t)kt * 4, Ssl((kt >> 2) & 1) + 4 * 64 * wave);
#pragma unroll
    for (int i = 0; i < NA; ++i)
      if (wave * RPW + i * 8 < mrows)  // rows past the segment feed no stored output
        load_lds16(g.A + a_off[i] + (uint32_t)kt * XBK, Asl(buf) + (wave * RPW + i * 8) * XBK);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if constexpr (B4)
        load_lds16(Bc + b_off[i] + (uint32_t)kt * (XBK / 2),
                   Bsl(buf) + (wave * RPW + i * 16) * BROW);
      else
        load_lds16(Bc + b_off[i] + (uint32_t)kt * XBK, Bsl(buf) + (wave * RPW + i * 8) * BROW);
    }
  };

  // ---- fragments and scales of the wave's blocks ------------------------------
  const int wm = wave / WCOLS, wn = wave % WCOLS;
  const int band = mrows - wm * 128;  // rows of this wave's 128-row band that exist
  const int lr = lane & 31, lh = lane >> 5;
  uint32_t sa[MI], sb[TJ];  // the lane's rows' (A) and columns' (B) scale words

  f32x16 acc[MI][TJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

  const int KT = K / XBK;
  gload(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  auto kloop = [&](auto skip_tag) {
    constexpr bool SK = decltype(skip_tag)::value;
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      // the other buffer was last read in step kt - 1, which every wave has left
      if (kt + 1 < KT) gload(kt + 1, cur ^ 1);
      {
        const uint32_t* S = g4 ? Ssl((kt >> 2) & 1) + (kt & 3) : Ssl(cur);
        const int rs = g4 ? 4 : 1;  // words per row
#pragma unroll
        for (int i = 0; i < MI; ++i) sa[i] = S[(wm * 128 + 32 * i + lr) * rs];
#pragma unroll
        for (int j = 0; j < TJ; ++j) sb[j] = S[(XBM + wn * WN + 32 * j + lr) * rs];
      }
      const uint8_t* Ab = Asl(cur) + (wm * 128) * XBK;
      const uint8_t* Bb = Bsl(cur) + (wn * WN) * BROW;
#pragma unroll
      for (int ks = 0; ks < XBK / 64; ++ks) {
        const int sh = 8 * (2 * ks + lh);  // this lane's K-block of the step
        v8i bf[TJ];
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int r = 32 * j + lr;
          const uint8_t* row = Bb + r * BROW;
          if constexpr (B4) {
            const uint4 w = *reinterpret_cast<const uint4*>(row + sw4(r, 2 * ks + lh) * 16);
            bf[j] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
          } else {
            const uint4 w0 = *reinterpret_cast<const uint4*>(row + sw8(r, 4 * ks + lh) * 16);
            const uint4 w1 = *reinterpret_cast<const uint4*>(row + sw8(r, 4 * ks + 2 + lh) * 16);
            bf[j] = v8i{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w,
                        (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
          }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if (SK && 32 * i >= band) continue;
          const int r = 32 * i + lr;
          const uint8_t* row = Ab + r * XBK;
          const uint4 w0 = *reinterpret_cast<const uint4*>(row + sw8(r, 4 * ks + lh) * 16);
          const uint4 w1 = *reinterpret_cast<const uint4*>(row + sw8(r, 4 * ks + 2 + lh) * 16);
          const v8i af = v8i{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w,
                             (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
          const int sai = (int)((sa[i] >> sh) & 0xffu);
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af, bf[j], acc[i][j], 0, B4 ? 4 : 0, 0, sai, 0, (int)((sb[j] >> sh) & 0xffu));
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of step kt + 1
      __syncthreads();
    }
  };
  if (band < MI * 32) kloop(std::integral_constant<bool, true>{});
  else kloop(std::integral_constant<bool, false>{});

  // ---- epilogue: acc[i][j][4 ii + jj] = C[row 32 i + 8 ii + 4 lh + jj][col 32 j + lr] ----
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int rloc = wm * 128 + 32 * i + 8 * ii + 4 * lh + jj;
        if (rloc >= mrows) continue;
        const long long m = m0 + rloc;
        if constexpr (EPI == MX_EPI_SWIGLU) {
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
            if (n < g.N) reinterpret_cast<float*>(g.out)[m * g.ldo + n] = acc[i][j][4 * ii + jj];
          }
        }
      }
}

static size_t mx_lds_bytes(bool b4) {
  return (size_t)2 * XBM * XBK + (size_t)2 * XBN * (b4 ? XBK / 2 : XBK) +
         (size_t)2 * 4 * (XBM + XBN) * 4;
}

template <int EPI, bool B4>
static int launch_mx(const MxGemmArgs& a, int max_mtiles, hipStream_t st) {
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_mx_kernel<EPI, B4>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)mx_lds_bytes(B4));
    attr = true;
  }
  hipLaunchKernelGGL((gemm_mx_kernel<EPI, B4>), dim3(max_mtiles * a.tiles_n), dim3(XWAVES * 64),
                     mx_lds_bytes(B4), st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int gemm_mx_rows() { return XBM; }

int launch_gemm_mx_swiglu(int F, int K, const uint8_t* A, const uint8_t* As,
                          const int32_t* gather, const uint8_t* B, const uint8_t* Bs, bool b4,
                          const int32_t* seg_off, const int32_t* tile_off, int E,
                          int max_mtiles, uint16_t* act, hipStream_t st) {
  if (K % XBK) return -1;
  MxGemmArgs a{};
  a.A = A; a.As = As; a.a_gather = gather; a.B = B; a.Bs = Bs;
  a.b_stride = (long long)2 * F * (b4 ? K / 2 : K);
  a.bs_stride = (long long)2 * F * (K / 32);
  a.N = 2 * F; a.K = K; a.seg_off = seg_off; a.tile_off = tile_off; a.E = E;
  a.tiles_n = (2 * F + XBN - 1) / XBN; a.out = act; a.ldo = F; a.F = F;
  return b4 ? launch_mx<MX_EPI_SWIGLU, true>(a, max_mtiles, st)
            : launch_mx<MX_EPI_SWIGLU, false>(a, max_mtiles, st);
}

int launch_gemm_mx_f32(int N, int K, const uint8_t* A, const uint8_t* As, const uint8_t* B,
                       const uint8_t* Bs, bool b4, const int32_t* seg_off,
                       const int32_t* tile_off, int E, int max_mtiles, float* out,
                       hipStream_t st) {
  if (K % XBK) return -1;
  MxGemmArgs a{};
  a.A = A; a.As = As; a.a_gather = nullptr; a.B = B; a.Bs = Bs;
  a.b_stride = (long long)N * (b4 ? K / 2 : K);
  a.bs_stride = (long long)N * (K / 32);
  a.N = N; a.K = K; a.seg_off = seg_off; a.tile_off = tile_off; a.E = E;
  a.tiles_n = (N + XBN - 1) / XBN; a.out = out; a.ldo = N; a.F = 0;
  return b4 ? launch_mx<MX_EPI_F32, true>(a, max_mtiles, st)
            : launch_mx<MX_EPI_F32, false>(a, max_mtiles, st);
}

}  // namespace beam
