// Many-token GQA attention over the KV cache (chunked prefill): causal inside
// the chunk, sliding window on SWA layers, full context on NoPE layers
// ("Reflection Beam 1.0 on vLLM", Attention section). The chunk's own keys
// were written to the cache first, so every token reads keys [lo_t, p_t] of
// its sequence from the cache alone.
//
// Workgroup = (block of 32*ntb consecutive tokens, kv head j): one wave per
// (query head of the group, 32-token sub-block), so every wave of the
// workgroup consumes the same keys. Keys advance in tiles of 64, staged
// cooperatively into a double-buffered LDS ring: the next tile's global loads
// are in flight while the current tile is multiplied out of LDS.
// attn_prefill_kernel (fp8 caches, which it widens exactly while staging, and
// head dims 32 / 64) holds K and V as bf16 and gives the P.V product each
// probability as a hi + lo pair of bf16 values (two MFMAs, ~16 bits):
//   S^T[key][token] = K[key][:] . Q[token][:]            32x32x16 bf16 MFMA
//   O^T[dim][token] += V^T[dim][key] . (P_hi + P_lo)^T    2 x 32x32x16 bf16 MFMA
// attn_prefill_dma_kernel (bf16 cache, head dim 128) takes the P.V product on
// fp16 operands instead, one MFMA: p (< 256: the running max only moves when
// a score passes it by more than 2^8) rounded to fp16 keeps 11 significant
// bits, and the bf16 V^T tile converts to fp16 exactly (values beyond +-65504
// are clamped).
// In the S^T layout lane l owns token l % 32: the online softmax state is
// lane-local up to one xor-32 shuffle, and a lane's probabilities are the B
// operand it needs for P.V. LDS rows are padded (K rows by 16 bytes, V^T rows
// by 8) so the fragment reads of consecutive rows hit distinct banks while
// every per-step offset stays an immediate. Value entries outside the tile's
// valid key range are zeroed while staged (they may hold anything).
// Tokens of several sequences in one block are handled in one pass per
// sequence.
#include "common.h"
#include "internal.h"

namespace beam {

BEAM_ERR_FLAG_DECL(attnp)
BEAM_ERR_FLAG_READER(attnp)

constexpr int KT = 64;  // keys per LDS tile

template <int HD, bool FP8, bool SWA>
__global__ __launch_bounds__(768) void attn_prefill_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ seq, const void* __restrict__ kc, const void* __restrict__ vc,
    int S, int Lmax, int npos, int Hq, int Hkv, int window, float score_scale, int T, int ntb,
    const float* __restrict__ sink, float v_scale, uint16_t* __restrict__ o) {
  constexpr int KS = HD / 16;    // k-steps of the score product
  constexpr int DB = HD / 32;    // 32-dim blocks of the output
  constexpr int LD = HD / 2;     // dims per lane half in the score product
  constexpr int KSTR = HD + 8;   // LDS row stride of K (bf16 elements)
  constexpr int VSTR = KT + 4;   // LDS row stride of V^T (bf16 elements)
  constexpr int NKU = KT * HD / 8;  // 8-element load units of a K tile
  constexpr int NU = NKU + HD * (KT / 8);
  extern __shared__ __align__(16) uint16_t lds[];
  // [K0 | K1 | V0 | V1]
  auto sK = [&](int b) { return lds + b * (KT * KSTR); };
  auto sV = [&](int b) { return lds + 2 * KT * KSTR + b * (HD * VSTR); };
  __shared__ int sinfo[3];

  const int nthr = blockDim.x, tid = threadIdx.x;
  const int j = blockIdx.y;
  const int grp = Hq / Hkv;
  const int wave = tid >> 6, lane = tid & 63;
  const int hh = wave % grp, tb = wave / grp;
  const int h = j * grp + hh;
  const int tc = lane & 31, g = lane >> 5;
  const int tblk = 32 * ntb;
  const int t0 = blockIdx.x * tblk;
  const int t = t0 + 32 * tb + tc;
  const bool tok = t < T;
  int p = tok ? pos[t] : -1, s = tok ? seq[t] : -1;
  if (p < 0 || p >= npos || s < 0 || s >= S) {
    if (tok && hh == 0) BEAM_RAISE(attnp, (p < 0 || p >= npos) ? ERR_POS : ERR_SEQ);
    p = -1;
    s = -1;
  }
  const int lo = SWA ? max(0, p - window + 1) : 0;

  bf16x8 qf[KS];
  if (p >= 0) {
    const uint16_t* qp = q + ((size_t)t * Hq + h) * HD + g * LD;
#pragma unroll
    for (int i = 0; i < KS; ++i) qf[i] = as_bf16x8(ld16(qp + i * 8));
  } else {
#pragma unroll
    for (int i = 0; i < KS; ++i) qf[i] = bf16x8{};
  }
  float m = -INFINITY, lsum = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  constexpr int UPT = 4;  // load units per thread per tile (NU <= UPT * 512)
  uint4 reg[UPT];

  int s_prev = -1;
  for (;;) {
    // ---- next sequence present in the block, and its key range ------------
    if (wave == 0) {
      int sc = 0x7fffffff;
      int tt = t0 + lane, pp = -1, ss = -1;
      if (lane < tblk && tt < T) {
        pp = pos[tt];
        ss = seq[tt];
        if (pp < 0 || pp >= npos || ss < 0 || ss >= S) ss = -1;
      }
      sc = (ss > s_prev) ? ss : 0x7fffffff;
      for (int o2 = 32; o2 > 0; o2 >>= 1) sc = min(sc, __shfl_xor(sc, o2, 64));
      const bool in = (ss == sc);
      int kmn = in ? (SWA ? max(0, pp - window + 1) : 0) : 0x7fffffff;
      int kmx = in ? pp : -1;
      for (int o2 = 32; o2 > 0; o2 >>= 1) {
        kmn = min(kmn, __shfl_xor(kmn, o2, 64));
        kmx = max(kmx, __shfl_xor(kmx, o2, 64));
      }
      if (lane == 0) {
        sinfo[0] = sc;
        sinfo[1] = kmn;
        sinfo[2] = kmx;
      }
    }
    __syncthreads();
    const int s_cur = sinfo[0], kmin = sinfo[1], kmax = sinfo[2];
    __syncthreads();
    if (s_cur == 0x7fffffff) break;
    s_prev = s_cur;
    const bool mine = (s == s_cur);
    const size_t krow0 = ((size_t)s_cur * Hkv + j) * (size_t)Lmax;
    const size_t vrow0 = ((size_t)s_cur * Hkv + j) * (size_t)HD;
    const int kb0 = kmin & ~(KT - 1);
    const int ntiles = (kmax - kb0) / KT + 1;

    auto gload = [&](int kb) {
      const int kbs = (npos > Lmax) ? kb % Lmax : kb;  // ring cache: slot of the first key
#pragma unroll
      for (int n = 0; n < UPT; ++n) {
        const int u = tid + n * nthr;
        if (u >= NU) break;
        if (u < NKU) {
          const int row = u / (HD / 8), c = u % (HD / 8);
          const size_t off = (krow0 + kbs + row) * HD + c * 8;
          if constexpr (FP8) {
            const uint2 w = *reinterpret_cast<const uint2*>((const uint8_t*)kc + off);
            reg[n] = uint4{w.x, w.y, 0u, 0u};
          } else {
            reg[n] = ld16((const uint16_t*)kc + off);
          }
        } else {
          const int u2 = u - NKU, dim = u2 >> 3, c = u2 & 7;
          const size_t off = (vrow0 + dim) * (size_t)Lmax + kbs + c * 8;
          if constexpr (FP8) {
            const uint2 w = *reinterpret_cast<const uint2*>((const uint8_t*)vc + off);
            reg[n] = uint4{w.x, w.y, 0u, 0u};
          } else {
            reg[n] = ld16((const uint16_t*)vc + off);
          }
        }
      }
    };
    auto lstore = [&](int buf, int kb) {
#pragma unroll
      for (int n = 0; n < UPT; ++n) {
        const int u = tid + n * nthr;
        if (u >= NU) break;
        if (u < NKU) {
          const int row = u / (HD / 8), c = u % (HD / 8);
          uint4 v = reg[n];
          if constexpr (FP8) v = __builtin_bit_cast(uint4, e4m3x8_to_bf16x8(uint2{v.x, v.y}));
          *reinterpret_cast<uint4*>(sK(buf) + row * KSTR + c * 8) = v;
        } else {
          const int u2 = u - NKU, dim = u2 >> 3, c = u2 & 7;
          bf16x8 hv;
          if constexpr (FP8) hv = e4m3x8_to_bf16x8(uint2{reg[n].x, reg[n].y});
          else hv = as_bf16x8(reg[n]);
          const int key = kb + c * 8;
          if (key < kmin || key + 7 > kmax) {  // edge tile: zero keys outside the range
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (key + e < kmin || key + e > kmax) hv[e] = (__bf16)0.0f;
          }
          uint16_t* vrow = sV(buf) + dim * VSTR + c * 8;
          const uint4 hb = __builtin_bit_cast(uint4, hv);
          *reinterpret_cast<uint2*>(vrow) = uint2{hb.x, hb.y};
          *reinterpret_cast<uint2*>(vrow + 4) = uint2{hb.z, hb.w};
        }
      }
    };

    gload(kb0);
    lstore(0, kb0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const int cur = it & 1;
      const int kb = kb0 + it * KT;
      if (it + 1 < ntiles) gload(kb + KT);
      if (__any(mine)) {  // waves with no token of this sequence only stage
#pragma unroll 1
        for (int kh = 0; kh < 2; ++kh) {
          const int kbase = kb + kh * 32;
          f32x16 sacc = f32x16{};
          const uint16_t* krow = sK(cur) + (kh * 32 + tc) * KSTR + g * LD;
#pragma unroll
          for (int i = 0; i < KS; ++i) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + i * 8);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[i], sacc, 0, 0, 0);
          }
          // sacc[4 i + jj] = S[key kbase + 8 i + 4 g + jj][token tc]
          float mx = -INFINITY;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int key = kbase + 8 * i + 4 * g + jj;
              float v = sacc[4 * i + jj] * score_scale;
              v = (!mine || key < lo || key > p) ? -INFINITY : v;
              sacc[4 * i + jj] = v;
              mx = fmaxf(mx, v);
            }
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          const float mn = fmaxf(m, mx);
          const float alpha = (mn == -INFINITY) ? 1.f : exp2f(m - mn);
          float rs = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float pr = (mn == -INFINITY) ? 0.f : exp2f(sacc[i] - mn);
            sacc[i] = pr;
            rs += pr;
          }
          rs += __shfl_xor(rs, 32, 64);
          lsum = lsum * alpha + rs;
          m = mn;
          if (__any(alpha != 1.f)) {  // rescale only when some running max moved
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
          }
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            bf16x8 ph, pl;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float pv = sacc[4 * (2 * st + (i >> 2)) + (i & 3)];
              ph[i] = (__bf16)pv;
              pl[i] = (__bf16)(pv - (float)ph[i]);
            }
            // this lane's keys: kh*32 + 16*st + 4*g + [0, 4) and the same + 8
            const uint16_t* vcol = sV(cur) + tc * VSTR + kh * 32 + 16 * st + 4 * g;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const uint2 a = *reinterpret_cast<const uint2*>(vcol + db * 32 * VSTR);
              const uint2 b = *reinterpret_cast<const uint2*>(vcol + db * 32 * VSTR + 8);
              const bf16x8 vf = __builtin_bit_cast(bf16x8, uint4{a.x, a.y, b.x, b.y});
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, ph, oacc[db], 0, 0, 0);
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl, oacc[db], 0, 0, 0);
            }
          }
        }
      }
      if (it + 1 < ntiles) lstore(cur ^ 1, kb + KT);
      __syncthreads();
    }
  }
  if (!tok || tb >= ntb) return;
  if (sink) {
    const float sl2 = sink[h] * 1.4426950408889634f;
    const float mn = fmaxf(m, sl2);
    const float a = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    lsum = lsum * a + exp2f(sl2 - mn);
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= a;
  }
  const float inv = (lsum > 0.f) ? v_scale / lsum : 0.f;
  uint16_t* op = o + ((size_t)t * Hq + h) * HD;
  // oacc[db][4 i + jj] = O[token tc][dim 32 db + 8 i + 4 g + jj]
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * db + 8 * i + 4 * g;
      uint2 w;
      w.x = pack_bf2(oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv);
      w.y = pack_bf2(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
      *reinterpret_cast<uint2*>(op + d0) = w;
    }
}

// ---------------------------------------------------------------------------
// bf16 cache, head dim 128: K and V^T tiles go from global memory straight into
// LDS (16 bytes per lane; one wave instruction fills 1 KiB), double-buffered,
// so no registers hold staged data and no padding is possible: bank conflicts
// are avoided with XOR swizzles instead. A 16-byte fragment read is served
// 16 lanes at a time (256 bytes: one line of the 64 banks).
//   K tile  [64 keys][128 dims]: row r = 16 chunks of 16 B, a full bank line;
//           chunk c of row r sits at slot c ^ fk(r), fk(r) = r & 15, so the
//           16 rows read by a group of 16 lanes (perm(0..15)) hit 16
//           distinct slots.
//   V^T tile [128 dims][64 keys]: row = 8 chunks (8 keys each), two rows per
//           bank line; chunk c of dim row d sits at slot c ^ ((d >> 1) & 7),
//           so the 8 rows of each parity among 16 consecutive dims get 8
//           distinct slots.
// The score MFMA takes key slot s of a 32-key half from K row perm(s), perm
// swapping bits 2 and 3, so that after the product lane (tc, g) holds the
// probabilities of keys 16 st + 8 g + [0, 8) for st = 0, 1: exactly one
// contiguous 16-byte V^T chunk per P.V step.
// Keys outside the sequence's [kmin, kmax] may hold anything: scores are
// replaced by -inf, and on edge tiles the out-of-range V^T entries are zeroed
// in LDS by the same pass that turns each V^T tile into fp16 (once per
// workgroup and tile, so the P.V loop carries no masking and no conversion):
//   O^T[dim][token] += V^T[dim][key] . P^T              32x32x16 fp16 MFMA
constexpr int DMA_HD = 128;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int fk_swz(int r) { return r & 15; }
__device__ __forceinline__ int fv_swz(int d) { return (d >> 1) & 7; }
__device__ __forceinline__ int perm23(int s) {
  return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1);
}
// max and sum of a value over lanes l and l ^ 32
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool SWA>
__global__ __launch_bounds__(768) void attn_prefill_dma_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ seq, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int S, int Lmax, int npos, int Hq, int Hkv, int window,
    float score_scale, int T, int ntb, const float* __restrict__ sink,
    uint16_t* __restrict__ o) {
  constexpr int HD = DMA_HD;
  constexpr int KS = HD / 16;  // k-steps of the score product
  constexpr int DB = HD / 32;  // 32-dim blocks of the output
  constexpr int LD = HD / 2;   // dims per lane half in the score product
  constexpr int TILE = KT * HD;              // elements of one K (or V^T) tile
  constexpr int NI = 2 * TILE * 2 / 1024;    // 1 KiB load instructions per tile pair (32)
  extern __shared__ __align__(16) uint16_t lds[];
  // [K0 | K1 | V0 | V1]
  auto sK = [&](int b) { return lds + b * TILE; };
  auto sV = [&](int b) { return lds + 2 * TILE + b * TILE; };
  __shared__ int sinfo[3];

  const int nw = blockDim.x >> 6, tid = threadIdx.x;
  // Workgroups are handed to the eight XCDs in turn: logical index L sends a
  // contiguous eighth of the (token block, kv head) grid to each XCD, so the
  // blocks that read one kv head's keys share that XCD's L2.
  const int nx = (int)gridDim.x, nwg = nx * (int)gridDim.y;
  const int b = (int)(blockIdx.y * gridDim.x + blockIdx.x);
  const int L = (nwg % 8 == 0) ? (b & 7) * (nwg >> 3) + (b >> 3) : b;
  const int xb = L % nx, j = L / nx;
  const int grp = Hq / Hkv;
  const int wave = tid >> 6, lane = tid & 63;
  const int hh = wave % grp, tb = wave / grp;
  const int h = j * grp + hh;
  const int tc = lane & 31, g = lane >> 5;
  const int tblk = 32 * ntb;
  const int t0 = xb * tblk;
  const int t = t0 + 32 * tb + tc;
  const bool tok = t < T;
  int p = tok ? pos[t] : -1, s = tok ? seq[t] : -1;
  if (p < 0 || p >= npos || s < 0 || s >= S) {
    if (tok && hh == 0) BEAM_RAISE(attnp, (p < 0 || p >= npos) ? ERR_POS : ERR_SEQ);
    p = -1;
    s = -1;
  }
  const int lo = SWA ? max(0, p - window + 1) : 0;

  bf16x8 qf[KS];
  if (p >= 0) {
    const uint16_t* qp = q + ((size_t)t * Hq + h) * HD + g * LD;
#pragma unroll
    for (int i = 0; i < KS; ++i) qf[i] = as_bf16x8(ld16(qp + i * 8));
  } else {
#pragma unroll
    for (int i = 0; i < KS; ++i) qf[i] = bf16x8{};
  }
  float m = -INFINITY, lsum = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  int s_prev = -1;
  for (;;) {
    // ---- next sequence present in the block, and its key range ------------
    if (wave == 0) {
      int tt = t0 + lane, pp = -1, ss = -1;
      if (lane < tblk && tt < T) {
        pp = pos[tt];
        ss = seq[tt];
        if (pp < 0 || pp >= npos || ss < 0 || ss >= S) ss = -1;
      }
      int sc = (ss > s_prev) ? ss : 0x7fffffff;
      for (int o2 = 32; o2 > 0; o2 >>= 1) sc = min(sc, __shfl_xor(sc, o2, 64));
      const bool in = (ss == sc);
      int kmn = in ? (SWA ? max(0, pp - window + 1) : 0) : 0x7fffffff;
      int kmx = in ? pp : -1;
      for (int o2 = 32; o2 > 0; o2 >>= 1) {
        kmn = min(kmn, __shfl_xor(kmn, o2, 64));
        kmx = max(kmx, __shfl_xor(kmx, o2, 64));
      }
      if (lane == 0) {
        sinfo[0] = sc;
        sinfo[1] = kmn;
        sinfo[2] = kmx;
      }
    }
    __syncthreads();
    const int s_cur = sinfo[0], kmin = sinfo[1], kmax = sinfo[2];
    __syncthreads();
    if (s_cur == 0x7fffffff) break;
    s_prev = s_cur;
    const bool mine = (s == s_cur);
    // a tile is interior for this wave when every token of the wave belongs to
    // this sequence and sees all 64 of its keys: no masking needed
    int p_min = mine ? p : 0x7fffffff, lo_max = mine ? lo : 0;
    for (int o2 = 32; o2 > 0; o2 >>= 1) {
      p_min = min(p_min, __shfl_xor(p_min, o2, 64));
      lo_max = max(lo_max, __shfl_xor(lo_max, o2, 64));
    }
    const bool all_mine = __all(mine);
    const uint16_t* kbase_p = kc + ((size_t)s_cur * Hkv + j) * (size_t)Lmax * HD;
    const uint16_t* vbase_p = vc + ((size_t)s_cur * Hkv + j) * (size_t)HD * Lmax;
    const int kb0 = kmin & ~(KT - 1);
    const int ntiles = (kmax - kb0) / KT + 1;

    // instruction u < 16: K rows 4u..4u+3; u >= 16: V^T dim rows 8(u-16)..+7.
    // kb + 63 <= Lmax - 1 for the tile's slot kb (64-aligned, below Lmax, and
    // Lmax % 64 == 0; on a ring cache, position kb mod Lmax).
    // Wave w issues units w, w + nw, ... (at most MAXU: nw >= 8); each lane's
    // address at key 0 is formed once per sequence, a tile adds kb to it.
    // (element offsets from the sequence's K / V^T base: d * Lmax < 2^31)
    constexpr int MAXU = 4;
    uint32_t go[MAXU];
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
      const int u = wave + i * nw;
      if (u < NI / 2) {
        const int r = 4 * u + (lane >> 4);
        go[i] = (uint32_t)(r * HD + ((lane & 15) ^ fk_swz(r)) * 8);
      } else {
        const int d = 8 * (u - NI / 2) + (lane >> 3);
        go[i] = (uint32_t)d * (uint32_t)Lmax + (uint32_t)(((lane & 7) ^ fv_swz(d)) * 8);
      }
    }
    auto gload = [&](int kb, int buf) {
      const int kbs = (npos > Lmax) ? kb % Lmax : kb;  // ring cache: slot of the first key
#pragma unroll
      for (int i = 0; i < MAXU; ++i) {
        const int u = wave + i * nw;
        if (u < NI / 2)
          load_lds16(kbase_p + (go[i] + (uint32_t)kbs * HD), sK(buf) + 4 * u * HD);
        else if (u < NI)
          load_lds16(vbase_p + (go[i] + (uint32_t)kbs), sV(buf) + 8 * (u - NI / 2) * KT);
      }
    };

    gload(kb0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const int cur = it & 1;
      const int kb = kb0 + it * KT;
      // the other buffer was last read in tile it - 1, which every wave has left
      if (it + 1 < ntiles) gload(kb + KT, cur ^ 1);
      const bool edge = (kb < kmin) || (kb + KT - 1 > kmax);
      const bool interior = all_mine && kb >= lo_max && kb + KT - 1 <= p_min;
      // The V^T tile becomes fp16 in place (the P.V product runs on fp16
      // operands: bf16 values in fp16's range convert exactly, larger ones are
      // clamped to +-65504 and reported), and on an edge tile the keys outside
      // the sequence's [kmin, kmax] become zero (they may hold anything).
      // Chunk slot s of V^T row d holds keys 8 (s ^ (d % 8)) + [0, 8) of the
      // tile.
      {
        uint4* vt = reinterpret_cast<uint4*>(sV(cur));
        uint32_t mag = 0;  // per 16-bit half: the largest fp16 magnitude written
        for (int c = tid; c < HD * KT / 8; c += nw * 64) {
          const uint4 w = vt[c];
          uint32_t in[4] = {w.x, w.y, w.z, w.w};
          if (edge) {
            const int d = c >> 3, k0 = kb + 8 * ((c & 7) ^ fv_swz(d));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (k0 + 2 * e < kmin || k0 + 2 * e > kmax) in[e] &= 0xffff0000u;
              if (k0 + 2 * e + 1 < kmin || k0 + 2 * e + 1 > kmax) in[e] &= 0x0000ffffu;
            }
          }
          uint32_t out[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // round toward zero: exact for bf16 values in fp16's range (but
            // those below 2^-17, off by under 2^-24), and an overflow gives
            // the largest finite value, +-65504
            out[e] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_pkrtz(bf_lo(in[e]), bf_hi(in[e])));
            // integer max per 16-bit half of the magnitudes written
            mag = __builtin_bit_cast(
                uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, mag),
                                                    __builtin_bit_cast(u16x2, out[e] & 0x7fff7fffu)));
          }
          vt[c] = uint4{out[0], out[1], out[2], out[3]};
        }
        // 65504 (0x7bff) is written only for a clamped value (no bf16 value
        // lies in [65504, 65536)); infinities and NaN (0x7c00 and up) are
        // reported with them
        if ((mag & 0xffffu) >= 0x7bffu || (mag >> 16) >= 0x7bffu) BEAM_RAISE(attnp, ERR_RANGE);
        __syncthreads();
      }
      if (__any(mine)) {  // waves with no token of this sequence only load
#pragma unroll 1
        for (int kh = 0; kh < 2; ++kh) {
          const int kbase = kb + kh * 32;
          f32x16 sacc = f32x16{};
          const int kr = kh * 32 + perm23(tc);
          const uint16_t* krow = sK(cur) + kr * HD;
#pragma unroll
          for (int i = 0; i < KS; ++i) {
            const int c = g * (LD / 8) + i;
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + (c ^ fk_swz(kr)) * 8);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[i], sacc, 0, 0, 0);
          }
          // sacc[4 i + jj] = S[key kbase + 16 (i >> 1) + 8 g + 4 (i & 1) + jj][token tc],
          // raw (unscaled) scores; m is the running max of raw scores (it only
          // moves when a score passes it by more than 2^8 in exp2 units, so the
          // probabilities stay below 256 and the output rescale is rare), and
          // the scale (> 0) enters once, inside exp2(s * c - m * c)
          if (!interior) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                const int key = kbase + 16 * (i >> 1) + 8 * g + 4 * (i & 1) + jj;
                if (!mine || key < lo || key > p) sacc[4 * i + jj] = -INFINITY;
              }
          }
          float mx = -INFINITY;
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
          mx = pair_max(mx);
          // also true when m is -inf and mx finite; false when both are -inf
          const bool grow = (mx - m) * score_scale > 8.f;
          const float mn = grow ? mx : m;
          const float moff = (mn == -INFINITY) ? 0.f : -mn * score_scale;
#pragma unroll
          for (int i = 0; i < 16; ++i)  // masked scores are -inf: exp2(-inf) = 0
            sacc[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], score_scale, moff));
          // p in fp16 (11 significant bits; p < 256): the P.V operand, and the
          // row sum taken over the same rounded values (two per dot instruction)
          f16x2 pp[2][4];
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int k = 0; k < 4; ++k)
              pp[st][k] = f16x2{(_Float16)sacc[4 * (2 * st + (k >> 1)) + 2 * (k & 1)],
                                (_Float16)sacc[4 * (2 * st + (k >> 1)) + 2 * (k & 1) + 1]};
          float rs = 0.f;
          const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int k = 0; k < 4; ++k) rs = __builtin_amdgcn_fdot2(pp[st][k], one2, rs, false);
          f16x8 pfs[2];
#pragma unroll
          for (int st = 0; st < 2; ++st)
            pfs[st] = __builtin_bit_cast(
                f16x8, uint4{__builtin_bit_cast(uint32_t, pp[st][0]),
                             __builtin_bit_cast(uint32_t, pp[st][1]),
                             __builtin_bit_cast(uint32_t, pp[st][2]),
                             __builtin_bit_cast(uint32_t, pp[st][3])});
          // lsum: this lane's share of the row sum (the two halves add up at
          // the end)
          if (__any(grow)) {  // rescale only when some running max moved
            // exp2(-inf) = 0 when nothing was accumulated yet
            const float alpha = grow ? __builtin_amdgcn_exp2f((m - mn) * score_scale) : 1.f;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
          }
          lsum += rs;
          m = mn;
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const f16x8 pf = pfs[st];
            // this lane's keys: kbase + 16 st + 8 g + [0, 8), one V^T chunk
            const int vchunk = kh * 4 + 2 * st + g;
            // the step's V^T fragments, all requested before the first product
            // (no masking here: an edge tile's out-of-range entries are zero)
            f16x8 vf[DB];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const int d = db * 32 + tc;
              vf[db] = *reinterpret_cast<const f16x8*>(sV(cur) + d * KT + (vchunk ^ fv_swz(d)) * 8);
            }
#pragma unroll
            for (int db = 0; db < DB; ++db)
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[db], pf, oacc[db], 0, 0, 0);
          }
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of tile it + 1
      __syncthreads();
    }
  }
  lsum = pair_sum(lsum);
  if (!tok || tb >= ntb) return;
  if (sink) {
    const float sl2 = sink[h] * 1.4426950408889634f;
    const float ms = (m == -INFINITY) ? -INFINITY : m * score_scale;  // log2 domain
    const float mn = fmaxf(ms, sl2);
    const float a = (m == -INFINITY) ? 0.f : exp2f(ms - mn);
    lsum = lsum * a + exp2f(sl2 - mn);
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= a;
  }
  const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
  uint16_t* op = o + ((size_t)t * Hq + h) * HD;
  // oacc[db][4 i + jj] = O[token tc][dim 32 db + 8 i + 4 g + jj]
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * db + 8 * i + 4 * g;
      uint2 w;
      w.x = pack_bf2(oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv);
      w.y = pack_bf2(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
      *reinterpret_cast<uint2*>(op + d0) = w;
    }
}

static size_t attn_prefill_lds(int hd) {
  return 2 * (size_t)KT * (hd + 8) * 2 + 2 * (size_t)hd * (KT + 4) * 2;
}

int launch_attn_prefill(int T, int Hq, int Hkv, int hd, int swa, int window, int fp8,
                        const uint16_t* q, const int32_t* pos, const int32_t* seq,
                        const void* kc, const void* vc, float k_scale, float v_scale, int S,
                        int Lmax, int npos, const float* sink, uint16_t* o, hipStream_t st) {
  const float score_scale = k_scale / sqrtf((float)hd) * 1.4426950408889634f;
  const int grp = Hq / Hkv;
  // waves per workgroup = grp * ntb <= 12; every thread stages at most 4 units
  // of 8 elements, so 256 * grp * ntb >= 16 * hd
  int ntb = (grp <= 6) ? 2 : 1;
  while (256 * grp * ntb < 16 * hd) ++ntb;
  if (grp * ntb > 12) return -1;
  const dim3 grid((T + 32 * ntb - 1) / (32 * ntb), Hkv), block(64 * grp * ntb);
  const float vs = fp8 ? v_scale : 1.0f;
  if (!fp8 && hd == DMA_HD) {
    const size_t sh = (size_t)4 * KT * DMA_HD * 2;
    auto go = [&](auto kern) {
      static bool attr = false;
      if (!attr) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
        attr = true;
      }
      hipLaunchKernelGGL(kern, grid, block, sh, st, q, pos, seq, (const uint16_t*)kc,
                         (const uint16_t*)vc, S, Lmax, npos, Hq, Hkv, window, score_scale, T, ntb,
                         sink, o);
    };
    if (swa) go(attn_prefill_dma_kernel<true>);
    else go(attn_prefill_dma_kernel<false>);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
#define PF(HD_, F8, SW)                                                                       \
  do {                                                                                         \
    const size_t sh = attn_prefill_lds(HD_);                                                   \
    static bool attr = false;                                                                  \
    if (!attr) {                                                                               \
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_prefill_kernel<HD_, F8, SW>), \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);          \
      attr = true;                                                                             \
    }                                                                                          \
    hipLaunchKernelGGL((attn_prefill_kernel<HD_, F8, SW>), grid, block, sh, st, q, pos, seq,  \
                       kc, vc, S, Lmax, npos, Hq, Hkv, window, score_scale, T, ntb, sink, vs, o); \
  } while (0)
#define BY_MODE(HD_)                                                  \
  if (fp8) {                                                         \
    if (swa) PF(HD_, true, true); else PF(HD_, true, false);         \
  } else {                                                           \
    if (swa) PF(HD_, false, true); else PF(HD_, false, false);       \
  }
  if (hd == 128) { BY_MODE(128) }
  else if (hd == 64) { BY_MODE(64) }
  else { BY_MODE(32) }
#undef BY_MODE
#undef PF
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace beam
