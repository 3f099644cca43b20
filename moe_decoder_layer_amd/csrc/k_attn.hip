// Decode-shaped GQA attention over the KV cache ("Reflection Beam 1.0 on
// vLLM", Attention section: 48 query heads share 8 kv heads, head dim 128;
// SWA layers see the last 512 positions, NoPE layers all of them).
//
// Split-K ("flash decoding"): workgroup (chunk c, kv head j, token t) covers
// 256*tpw keys of the token's visible range, each of its 4 waves a run of tpw
// tiles of 64 keys. Per tile and wave, on the matrix cores:
//   S^T[key][head] = K[key][:] . Q[head][:]   16x16x32 bf16 MFMA, the GQA group
//                                             (<= 16 query heads) is the N axis
//   O^T[dim][head] += V^T[dim][key] . P^T[key][head]
// With S^T in the C layout, lane l owns query head l%16 for 16 keys, so the
// online-softmax state (m, l) of a head is lane-local up to two xor shuffles,
// and the probabilities a lane holds are exactly the keys it needs as the B
// operand of the P.V product (no LDS round trip). The score product takes its
// keys in a permuted slot order that makes those 8 keys consecutive, and V is
// stored transposed in the cache, so each lane's V operand is one contiguous
// load.
// fp8 caches are widened to bf16 exactly with gfx950's packed conversion; the
// per-tensor scales are applied to the scores (k) and the output (v).
// Probabilities enter the P.V product as hi + lo bf16 pairs (two MFMAs), so
// the only bf16 rounding of the attention path is its output.
// Each wave's (m, l, O) is merged in LDS; one fp32 record per (t, head, c) goes
// to the workspace. The chunks of a (token, kv head) are combined by the last
// of its workgroups to finish when there are few of them, else by
// attn_merge_kernel; a span that fits one workgroup is normalised in place.
#include "common.h"
#include "internal.h"
#include "qk_head.h"

namespace beam {

BEAM_ERR_FLAG_DECL(attn)
BEAM_ERR_FLAG_READER(attn)

// NW waves per workgroup; GS query-head slots kept for the LDS merge (>= group).
// Split-K workgroups take contiguous runs of tpw tiles per wave; a one-pass
// workgroup (o_direct != nullptr) deals the span's tiles round-robin to its
// waves so no wave walks more than ceil(tiles / NW) of them. With ctr set, the
// last workgroup of each (token, kv head) to finish merges its chunks and
// writes o_direct (ctr[t * Hkv + j] counts arrivals and is left at zero).
// Lane group g holds, in k-step i of the score product, the 8 dims from
// qk_dim(i, g) on (the same for the query and the key operand). With these
// runs, one 16-byte load per lane covers 64 contiguous bytes of each of 16 key
// rows across the four lane groups.
template <int HD, bool FP8>
__device__ __forceinline__ constexpr int qk_dim(int i, int g) {
  if constexpr (FP8) return HD >= 64 ? (i >> 1) * 64 + g * 16 + (i & 1) * 8 : g * 8;
  return i * 32 + g * 8;
}

// Key, within a 64-key tile, of score slot 4 q4 + r of block st. Lane group g
// then holds the probabilities of keys half_key(kh, g) + [0, 8) for kh = 0, 1,
// i.e. exactly its B operand of the two P.V steps, and the matching V^T runs
// are contiguous across the lane groups (16 keys per lane for fp8: one
// 16-byte load; 8 keys per half for bf16).
template <bool FP8>
__device__ __forceinline__ constexpr int slot_key(int st, int q4, int r) {
  return FP8 ? 16 * q4 + 8 * (st >> 1) + 4 * (st & 1) + r
             : 32 * (st >> 1) + 8 * q4 + 4 * (st & 1) + r;
}
template <bool FP8>
__device__ __forceinline__ constexpr int half_key(int kh, int g) {
  return FP8 ? 16 * g + 8 * kh : 32 * kh + 8 * g;
}

// Replace element e of a 16-byte fragment (8 bf16 values / 16 fp8 codes).
__device__ __forceinline__ void frag_set_u16(uint4& v, int e, uint16_t x) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (e == 2 * i) w[i] = (w[i] & 0xffff0000u) | x;
    if (e == 2 * i + 1) w[i] = (w[i] & 0x0000ffffu) | ((uint32_t)x << 16);
  }
  v = uint4{w[0], w[1], w[2], w[3]};
}
__device__ __forceinline__ void frag_set_u8(uint4& v, int e, uint8_t x) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (e == i) w[i >> 2] = (w[i >> 2] & ~(0xffu << (8 * (i & 3)))) | ((uint32_t)x << (8 * (i & 3)));
  v = uint4{w[0], w[1], w[2], w[3]};
}

// The attention output element o (fp32) as stored with the output gate:
// bf16(bf16(o) * sigmoid(g + b)), the gate formed exactly as the o_proj call's
// gate prologue forms it (g: the gate projection's bf16 value, b: the head's
// bias).
__device__ __forceinline__ uint16_t attn_out_gated(float o, uint16_t g, float b) {
  return f2bf(round_bf(o) * sigmoidf_fast(bf2f(g) + b));
}

template <int HD, bool FP8, bool SWA, int NW, int GS, bool FUSED>
__device__ __forceinline__ void attn_decode_body(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ seq, const void* __restrict__ kc, const void* __restrict__ vc,
    int S, int Lmax, int npos, int Hq, int Hkv, int window, int tpw, float score_scale,
    int nch_stride, float* part, uint16_t* __restrict__ o_direct, const float* __restrict__ sink,
    float v_scale, unsigned* ctr, const AttnFuse fz) {
  constexpr int KS = HD / 32;  // k-steps of the score product
  constexpr int DT = HD / 16;  // 16-dim tiles of the output
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ float sm_o[NW][GS][HD + 4];
  __shared__ int s_last;
  // FUSED: the group's normed q, and the new key and value (bf16 bits, or
  // fp8 codes in the first HD bytes)
  __shared__ __align__(16) uint16_t sq[FUSED ? GS : 1][FUSED ? HD : 8];
  __shared__ __align__(16) uint16_t skv[FUSED ? 2 : 1][FUSED ? HD : 8];
  // FUSED with the output gate: the group's gate values and biases
  __shared__ uint16_t sg[FUSED ? GS * HD : 1];
  __shared__ float sbg[FUSED ? GS : 1];

  const int c = blockIdx.x, j = blockIdx.y, t = blockIdx.z;
  const int grp = Hq / Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;

  // FUSED: the gate values this workgroup may need at its merge are requested
  // first (they reach LDS with the epilogue's barrier), so the merge does not
  // wait on them
  constexpr int GPT = FUSED ? (GS * HD + NW * 64 - 1) / (NW * 64) : 1;
  uint16_t gpre[GPT];
  float bpre = 0.f;
  const bool gated = FUSED && fz.g != nullptr;
  if (gated) {
#pragma unroll
    for (int k = 0; k < GPT; ++k) {
      const int i = threadIdx.x + k * NW * 64;
      gpre[k] = i < grp * HD ? fz.g[((size_t)t * Hq + j * grp) * HD + i] : 0;
    }
    if ((int)threadIdx.x < grp) bpre = bf2f(fz.bgate[j * grp + threadIdx.x]);
  }
  // the query fragments do not depend on the position: request them first
  // (FUSED: formed below from the raw projection)
  bf16x8 qf[KS];
  if (FUSED) {
#pragma unroll
    for (int i = 0; i < KS; ++i) qf[i] = bf16x8{};
  } else if (col < grp) {
    const uint16_t* qp = q + ((size_t)t * Hq + j * grp + col) * HD;
#pragma unroll
    for (int i = 0; i < KS; ++i) qf[i] = as_bf16x8(ld16(qp + qk_dim<HD, FP8>(i, g)));
  } else {
#pragma unroll
    for (int i = 0; i < KS; ++i) qf[i] = bf16x8{};
  }

  const int p = pos[t], s = seq[t];
  const int CK = NW * 64 * tpw;
  int bad = (p < 0 || p >= npos) ? ERR_POS : (s < 0 || s >= S) ? ERR_SEQ : 0;
  int lo = 0, nch = 0;
  if (!bad) {
    lo = SWA ? max(0, p - window + 1) : 0;
    nch = (p + 1 - (lo & ~63) + CK - 1) / CK;
    // a position beyond the host's max_pos needs more chunks than the grid
    // and the record stride were sized for: none of them runs (so no arrival
    // is counted and no record is written out of place)
    if (nch > nch_stride) bad = ERR_SPAN;
  }
  if (bad) {
    if (c == 0 && j == 0 && threadIdx.x == 0) BEAM_RAISE(attn, bad);
    if (o_direct && c == 0)
      for (int i = threadIdx.x; i < grp * HD; i += NW * 64)
        o_direct[((size_t)t * Hq + j * grp) * HD + i] = 0;
    return;
  }
  const int lo_al = lo & ~63;
  if (c >= nch) return;

  // Position k lives in slot k mod Lmax (the identity unless the cache is a
  // ring, npos > Lmax); a 64-key tile never wraps (Lmax % 64 == 0).
  const bool ring = npos > Lmax;
  const int ps = ring ? p % Lmax : p;                          // slot of position p
  const size_t krow0 = ((size_t)s * Hkv + j) * (size_t)Lmax;  // K row of slot 0
  const size_t vrow0 = ((size_t)s * Hkv + j) * (size_t)HD;    // V^T row of dim 0
  float m = -INFINITY, lsum = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool rr = (o_direct != nullptr) && (ctr == nullptr);
  const int tile0 = (lo_al >> 6) + (rr ? wave : (c * NW + wave) * tpw);
  // The tile's K and V fragments are all requested before any is used (key
  // slots permuted by slot_key, dims by qk_dim). Fragments stay in their
  // stored form (fp8 codes: half the registers) until the product that uses
  // them.
  constexpr int KR = FP8 ? (KS + 1) / 2 : KS;  // 16-byte K loads per slot
  constexpr int VR = FP8 ? 1 : 2;              // 16-byte V loads per output tile
  uint4 kraw[4][KR];
  uint4 vraw[DT][VR];
  auto load_tile = [&](int kb) {
    const int kbs = ring ? kb % Lmax : kb;  // slot of the tile's first key
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int key = kbs + slot_key<FP8>(st, col >> 2, col & 3);
      const size_t kr = (krow0 + key) * HD;
      if constexpr (FP8 && KS >= 2) {  // steps 2h, 2h+1 share one 16-byte load
#pragma unroll
        for (int i = 0; i < KR; ++i)
          kraw[st][i] = ld16((const uint8_t*)kc + kr + qk_dim<HD, FP8>(2 * i, g));
      } else if constexpr (FP8) {
        const uint2 w =
            *reinterpret_cast<const uint2*>((const uint8_t*)kc + kr + qk_dim<HD, FP8>(0, g));
        kraw[st][0] = uint4{w.x, w.y, 0u, 0u};
      } else {
#pragma unroll
        for (int i = 0; i < KS; ++i)
          kraw[st][i] = ld16((const uint16_t*)kc + kr + qk_dim<HD, FP8>(i, g));
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const size_t vr = (vrow0 + dt * 16 + col) * (size_t)Lmax + kbs;
      if constexpr (FP8) {
        vraw[dt][0] = ld16((const uint8_t*)vc + vr + half_key<FP8>(0, g));
      } else {
        vraw[dt][0] = ld16((const uint16_t*)vc + vr + half_key<FP8>(0, g));
        vraw[dt][1] = ld16((const uint16_t*)vc + vr + half_key<FP8>(1, g));
      }
    }
  };
  const bool has_p = FUSED && (c == nch - 1);  // this workgroup's span ends at p
  if constexpr (FUSED) {
    // The first tile is requested, then the epilogue of the projection runs
    // while it is in flight: the group's q heads (norm, RoPE or SSMax) into
    // LDS (chunk 0 also stores them), and in the workgroup whose span holds
    // position p the new key (norm, RoPE) and value, into LDS and the cache.
    // No other workgroup reads slot p; this one takes the new key and value
    // from LDS in place of the slot's old contents.
    const int kb0 = tile0 << 6;
    if (kb0 <= p) load_tile(kb0);
    const int nheads = Hq + 2 * Hkv;
    const uint16_t* row = fz.qkv + (size_t)t * nheads * HD;
    const int half = HD / 2;
    const int nitems = grp + (has_p ? 2 : 0);
    for (int u = wave; u < nitems; u += NW) {
      if (u < grp) {
        const int h = j * grp + u;
        float a, b;
        qk_head_pair(row + (size_t)h * HD, true, HD, fz.wq, fz.wk, p, true, fz.mode, fz.rope,
                     fz.eps, a, b);
        if (lane < half) {
          const uint16_t ba = f2bf(a), bb = f2bf(b);
          sq[u][lane] = ba;
          sq[u][lane + half] = bb;
          if (fz.q_out && c == 0) {
            fz.q_out[((size_t)t * Hq + h) * HD + lane] = ba;
            fz.q_out[((size_t)t * Hq + h) * HD + lane + half] = bb;
          }
        }
      } else if (u == grp) {  // the new key: K[s][j][p][:]
        float a, b;
        qk_head_pair(row + (size_t)(Hq + j) * HD, false, HD, fz.wq, fz.wk, p, true, fz.mode,
                     fz.rope, fz.eps, a, b);
        if (lane < half) {
          const size_t kr = (krow0 + ps) * HD;
          if constexpr (FP8) {
            uint8_t* k8 = reinterpret_cast<uint8_t*>(skv[0]);
            const uint8_t ca = f2e4m3(__fdiv_rn(a, fz.ks)), cb = f2e4m3(__fdiv_rn(b, fz.ks));
            k8[lane] = ca;
            k8[lane + half] = cb;
            ((uint8_t*)kc)[kr + lane] = ca;
            ((uint8_t*)kc)[kr + lane + half] = cb;
          } else {
            const uint16_t ba = f2bf(a), bb = f2bf(b);
            skv[0][lane] = ba;
            skv[0][lane + half] = bb;
            ((uint16_t*)kc)[kr + lane] = ba;
            ((uint16_t*)kc)[kr + lane + half] = bb;
          }
        }
      } else if (lane < half) {  // the new value, as produced: V^T[s][j][:][p]
        const uint16_t* vsrc = row + (size_t)(Hq + Hkv + j) * HD;
        const uint16_t va = vsrc[lane], vb = vsrc[lane + half];
        const size_t ca0 = (vrow0 + lane) * (size_t)Lmax + ps;
        const size_t cb0 = (vrow0 + lane + half) * (size_t)Lmax + ps;
        if constexpr (FP8) {
          uint8_t* v8 = reinterpret_cast<uint8_t*>(skv[1]);
          const uint8_t ca = f2e4m3(__fdiv_rn(bf2f(va), fz.vs));
          const uint8_t cb = f2e4m3(__fdiv_rn(bf2f(vb), fz.vs));
          v8[lane] = ca;
          v8[lane + half] = cb;
          ((uint8_t*)vc)[ca0] = ca;
          ((uint8_t*)vc)[cb0] = cb;
        } else {
          skv[1][lane] = va;
          skv[1][lane + half] = vb;
          ((uint16_t*)vc)[ca0] = va;
          ((uint16_t*)vc)[cb0] = vb;
        }
      }
    }
    if (gated) {
#pragma unroll
      for (int k = 0; k < GPT; ++k) {
        const int i = threadIdx.x + k * NW * 64;
        if (i < grp * HD) sg[i] = gpre[k];
      }
      if ((int)threadIdx.x < grp) sbg[threadIdx.x] = bpre;
    }
    __syncthreads();
    if (col < grp) {
#pragma unroll
      for (int i = 0; i < KS; ++i)
        qf[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&sq[col][qk_dim<HD, FP8>(i, g)]));
    }
  }
  // FUSED: the new key and value replace slot p's stale contents in the
  // fragments of the tile that holds p
  auto patch_tile = [&](int kb) {
    const uint8_t* k8 = reinterpret_cast<const uint8_t*>(skv[0]);
    const uint8_t* v8 = reinterpret_cast<const uint8_t*>(skv[1]);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (kb + slot_key<FP8>(st, col >> 2, col & 3) != p) continue;
      if constexpr (FP8 && KS >= 2) {
#pragma unroll
        for (int i = 0; i < KR; ++i)
          kraw[st][i] = *reinterpret_cast<const uint4*>(k8 + qk_dim<HD, FP8>(2 * i, g));
      } else if constexpr (FP8) {
        const uint2 w = *reinterpret_cast<const uint2*>(k8 + qk_dim<HD, FP8>(0, g));
        kraw[st][0] = uint4{w.x, w.y, 0u, 0u};
      } else {
#pragma unroll
        for (int i = 0; i < KS; ++i)
          kraw[st][i] = *reinterpret_cast<const uint4*>(&skv[0][qk_dim<HD, FP8>(i, g)]);
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dim = dt * 16 + col;
      if constexpr (FP8) {
        const int e = p - (kb + half_key<FP8>(0, g));
        if (e >= 0 && e < 16) frag_set_u8(vraw[dt][0], e, v8[dim]);
      } else {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int e = p - (kb + half_key<FP8>(kh, g));
          if (e >= 0 && e < 8) frag_set_u16(vraw[dt][kh], e, skv[1][dim]);
        }
      }
    }
  };
  for (int it = 0; it < tpw; ++it) {
    const int kb = (tile0 + (rr ? it * NW : it)) << 6;
    if (kb > p) break;
    if (!FUSED || it > 0) load_tile(kb);
    if (has_p && kb <= p && p < kb + 64) patch_tile(kb);
    f32x4 sacc[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      sacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        bf16x8 kf;
        if constexpr (FP8) {
          const uint4 w = kraw[st][i >> 1];
          kf = e4m3x8_to_bf16x8((i & 1) ? uint2{w.z, w.w} : uint2{w.x, w.y});
        } else {
          kf = as_bf16x8(kraw[st][i]);
        }
        sacc[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[i], sacc[st], 0, 0, 0);
      }
    }
    // scores (log2 domain), window mask, online softmax
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + slot_key<FP8>(st, g, r);
        float v = sacc[st][r] * score_scale;
        v = (key < lo || key > p) ? -INFINITY : v;
        sacc[st][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);  // finite: each visited tile holds a key in [lo, p]
    const float alpha = exp2f(m - mn);
    float rs = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = exp2f(sacc[st][r] - mn);
        sacc[st][r] = pr;
        rs += pr;
      }
    rs += __shfl_xor(rs, 16, 64);
    rs += __shfl_xor(rs, 32, 64);
    lsum = lsum * alpha + rs;
    m = mn;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;

    const bool edge = (kb < lo) || (kb + 63 > p);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      // P as a sum of two bf16 parts (hi + lo): the product keeps ~16 bits of
      // each probability instead of 8, at the cost of a second MFMA per tile
      bf16x8 pf, pl;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = sacc[2 * kh + (i >> 2)][i & 3];
        pf[i] = (__bf16)pv;
        pl[i] = (__bf16)(pv - (float)pf[i]);
      }
      const int key0 = kb + half_key<FP8>(kh, g);  // this lane's keys key0 + [0, 8)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x8 vf;
        if constexpr (FP8) {
          const uint4 w = vraw[dt][0];
          vf = e4m3x8_to_bf16x8(kh ? uint2{w.z, w.w} : uint2{w.x, w.y});
        } else {
          vf = as_bf16x8(vraw[dt][kh]);
        }
        if (edge) {  // keys outside [lo, p] may hold anything: zero them
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (key0 + i < lo || key0 + i > p) vf[i] = (__bf16)0.0f;
        }
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl, o[dt], 0, 0, 0);
      }
    }
  }

  if (g == 0) {
    sm_m[wave][col] = m;
    sm_l[wave][col] = lsum;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (col < GS) sm_o[wave][col][dt * 16 + 4 * g + r] = o[dt][r];
  __syncthreads();
  for (int i = threadIdx.x; i < grp * HD; i += NW * 64) {
    const int hh = i / HD, dim = i - hh * HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][hh]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float e = (sm_m[w][hh] == -INFINITY) ? 0.f : exp2f(sm_m[w][hh] - M);
      L += e * sm_l[w][hh];
      O += e * sm_o[w][hh][dim];
    }
    if (rr) {  // the whole span was this workgroup's: normalise and store
      if (sink) {
        const float sl2 = sink[j * grp + hh] * 1.4426950408889634f;
        const float Mn = fmaxf(M, sl2);
        const float a = exp2f(M - Mn);
        L = L * a + exp2f(sl2 - Mn);
        O *= a;
      }
      const size_t oi = ((size_t)t * Hq + j * grp + hh) * HD + dim;
      o_direct[oi] = gated ? attn_out_gated(O * (v_scale / L), sg[hh * HD + dim], sbg[hh])
                           : f2bf(O * (v_scale / L));
      continue;
    }
    float* rec = part + (((size_t)t * Hq + j * grp + hh) * nch_stride + c) * (HD + 4);
    if (dim == 0) {
      st_dev(rec, M);
      st_dev(rec + 1, L);
    }
    st_dev(rec + 4 + dim, O);
  }
  if (ctr == nullptr || !last_arrival(ctr + (size_t)t * Hkv + j, nch, &s_last)) return;
  // Last of the token's nch (<= kAttnFusedMergeMax) workgroups for this kv
  // head: wave w combines heads w, w + NW, ... in chunk order, with every
  // chunk's record requested before any is used.
  constexpr int MX = kAttnFusedMergeMax;
  constexpr int DPL = (HD + 63) / 64;  // dims per lane
  for (int hh = wave; hh < grp; hh += NW) {
    const float* rec0 = part + ((size_t)t * Hq + j * grp + hh) * nch_stride * (HD + 4);
    float mc[MX], lc[MX], oc[MX][DPL];
#pragma unroll
    for (int cc = 0; cc < MX; ++cc) {
      const float* rec = rec0 + (size_t)min(cc, nch - 1) * (HD + 4);
      mc[cc] = rec[0];
      lc[cc] = rec[1];
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int d = lane + 64 * k;
        oc[cc][k] = d < HD ? rec[4 + d] : 0.f;
      }
    }
    float M = -INFINITY;
#pragma unroll
    for (int cc = 0; cc < MX; ++cc)
      if (cc < nch) M = fmaxf(M, mc[cc]);
    const float sl2 = sink ? sink[j * grp + hh] * 1.4426950408889634f : -INFINITY;
    M = fmaxf(M, sl2);
    float L = sink ? exp2f(sl2 - M) : 0.f;
    float O[DPL] = {};
#pragma unroll
    for (int cc = 0; cc < MX; ++cc) {
      if (cc < nch) {
        const float e = exp2f(mc[cc] - M);
        L += e * lc[cc];
#pragma unroll
        for (int k = 0; k < DPL; ++k) O[k] += e * oc[cc][k];
      }
    }
    const float inv = v_scale / L;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int d = lane + 64 * k;
      const size_t oi = ((size_t)t * Hq + j * grp + hh) * HD + d;
      if (d < HD)
        o_direct[oi] = gated ? attn_out_gated(O[k] * inv, sg[hh * HD + d], sbg[hh])
                             : f2bf(O[k] * inv);
    }
  }
}

#define ATTN_DECODE_PARAMS                                                                    \
  const uint16_t *__restrict__ q, const int32_t *__restrict__ pos,                          \
      const int32_t *__restrict__ seq, const void *__restrict__ kc,                         \
      const void *__restrict__ vc, int S, int Lmax, int npos, int Hq, int Hkv, int window,  \
      int tpw, float score_scale, int nch_stride, float *part,                              \
      uint16_t *__restrict__ o_direct,                                                      \
      const float *__restrict__ sink, float v_scale, unsigned *ctr, const AttnFuse fz
#define ATTN_DECODE_ARGS                                                                 \
  q, pos, seq, kc, vc, S, Lmax, npos, Hq, Hkv, window, tpw, score_scale, nch_stride, part,    \
      o_direct,                                                                              \
      sink, v_scale, ctr, fz

template <int HD, bool FP8, bool SWA, int NW, int GS, bool FUSED>
__global__ __launch_bounds__(NW * 64) void attn_decode_partial_kernel(ATTN_DECODE_PARAMS) {
  attn_decode_body<HD, FP8, SWA, NW, GS, FUSED>(ATTN_DECODE_ARGS);
}

// Long split-K spans over an fp8 cache: the register budget is held to three
// waves per SIMD (from two), which keeps more of the cache stream in flight.
template <int HD, bool SWA, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void
attn_decode_fp8_stream_kernel(ATTN_DECODE_PARAMS) {
  attn_decode_body<HD, true, SWA, 4, 16, FUSED>(ATTN_DECODE_ARGS);
}

// The same combine for spans of at most kAttnFusedMergeMax chunks, one wave
// per (token, head), four per workgroup: every record requested before use.
template <int HD>
__global__ __launch_bounds__(256) void attn_merge_small_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ seq, int S, int npos, int T, int Hq, int window, int swa,
    int tpw, int nch_stride, const float* __restrict__ sink, float v_scale,
    uint16_t* __restrict__ o, const uint16_t* __restrict__ G, const uint16_t* __restrict__ bgate) {
  constexpr int MX = kAttnFusedMergeMax;
  constexpr int DPL = (HD + 63) / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int u = blockIdx.x * 4 + wave;
  if (u >= T * Hq) return;
  const int t = u / Hq, h = u - t * Hq;
  uint16_t* out = o + (size_t)u * HD;
  uint16_t gp[DPL] = {};  // the output gate's inputs, requested first
  float bp = 0.f;
  if (G) {
#pragma unroll
    for (int k = 0; k < DPL; ++k)
      if (lane + 64 * k < HD) gp[k] = G[(size_t)u * HD + lane + 64 * k];
    bp = bf2f(bgate[h]);
  }
  const int p = pos[t], s = seq[t];
  if (p < 0 || p >= npos || s < 0 || s >= S) {
    for (int d = lane; d < HD; d += 64) out[d] = 0;
    return;
  }
  const int lo = swa ? max(0, p - window + 1) : 0;
  const int CK = 256 * tpw;
  const int nch = (p + 1 - (lo & ~63) + CK - 1) / CK;
  if (nch > nch_stride) {  // beyond max_pos: flagged by the partial kernel, no records
    for (int d = lane; d < HD; d += 64) out[d] = 0;
    return;
  }
  const float* rec0 = part + (size_t)u * nch_stride * (HD + 4);
  float mc[MX], lc[MX], oc[MX][DPL];
#pragma unroll
  for (int c = 0; c < MX; ++c) {
    const float* rec = rec0 + (size_t)min(c, nch - 1) * (HD + 4);
    mc[c] = rec[0];
    lc[c] = rec[1];
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int d = lane + 64 * k;
      oc[c][k] = d < HD ? rec[4 + d] : 0.f;
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < MX; ++c)
    if (c < nch) M = fmaxf(M, mc[c]);
  const float sl2 = sink ? sink[h] * 1.4426950408889634f : -INFINITY;
  M = fmaxf(M, sl2);
  float L = sink ? exp2f(sl2 - M) : 0.f;
  float O[DPL] = {};
#pragma unroll
  for (int c = 0; c < MX; ++c) {
    if (c < nch) {
      const float e = exp2f(mc[c] - M);
      L += e * lc[c];
#pragma unroll
      for (int k = 0; k < DPL; ++k) O[k] += e * oc[c][k];
    }
  }
  const float inv = v_scale / L;
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int d = lane + 64 * k;
    if (d < HD) out[d] = G ? attn_out_gated(O[k] * inv, gp[k], bp) : f2bf(O[k] * inv);
  }
}

// Combine the chunks of one (token, head): o = sum_c 2^(m_c-M) O_c / sum_c 2^(m_c-M) l_c.
// An attention sink adds 2^(sink*log2e - M) to the denominator only. Wave w
// takes chunks w, w + MW, ... in batches of 8 whose records are all requested
// before use, keeping a running (M, L, O); the MW waves combine through LDS.
template <int HD>
__global__ __launch_bounds__(1024) void attn_merge_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ seq, int S, int npos, int Hq, int window, int swa, int tpw,
    int nch_stride, const float* __restrict__ sink, float v_scale, uint16_t* __restrict__ o,
    const uint16_t* __restrict__ G, const uint16_t* __restrict__ bgate) {
  constexpr int DPL = (HD + 63) / 64;
  constexpr int B = 8;
  constexpr int MW = 16;  // waves
  __shared__ float sm_m[MW], sm_l[MW], sm_o[MW][HD];
  const int h = blockIdx.x, t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint16_t* out = o + ((size_t)t * Hq + h) * HD;
  uint16_t gp[DPL] = {};  // the output gate's inputs (wave 0 stores), requested first
  float bp = 0.f;
  if (G && wave == 0) {
#pragma unroll
    for (int k = 0; k < DPL; ++k)
      if (lane + 64 * k < HD) gp[k] = G[((size_t)t * Hq + h) * HD + lane + 64 * k];
    bp = bf2f(bgate[h]);
  }
  const int p = pos[t], s = seq[t];
  if (p < 0 || p >= npos || s < 0 || s >= S) {
    for (int d = threadIdx.x; d < HD; d += MW * 64) out[d] = 0;
    return;
  }
  const int lo = swa ? max(0, p - window + 1) : 0;
  const int lo_al = lo & ~63;
  const int CK = 256 * tpw;
  const int nch = (p + 1 - lo_al + CK - 1) / CK;
  if (nch > nch_stride) {  // beyond max_pos: flagged by the partial kernel, no records
    for (int d = threadIdx.x; d < HD; d += MW * 64) out[d] = 0;
    return;
  }
  const float* rec0 = part + ((size_t)t * Hq + h) * nch_stride * (HD + 4);
  float M = -INFINITY, L = 0.f, O[DPL] = {};
  for (int c0 = wave; c0 < nch; c0 += MW * B) {
    float mc[B], lc[B], oc[B][DPL];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float* rec = rec0 + (size_t)min(c0 + MW * b, nch - 1) * (HD + 4);
      mc[b] = rec[0];
      lc[b] = rec[1];
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int d = lane + 64 * k;
        oc[b][k] = d < HD ? rec[4 + d] : 0.f;
      }
    }
    float Mn = M;
#pragma unroll
    for (int b = 0; b < B; ++b)
      if (c0 + MW * b < nch) Mn = fmaxf(Mn, mc[b]);
    const float a = exp2f(M - Mn);  // M = -inf on the first batch: a = 0
    L *= a;
#pragma unroll
    for (int k = 0; k < DPL; ++k) O[k] *= a;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (c0 + MW * b < nch) {
        const float e = exp2f(mc[b] - Mn);
        L += e * lc[b];
#pragma unroll
        for (int k = 0; k < DPL; ++k) O[k] += e * oc[b][k];
      }
    }
    M = Mn;
  }
  if (lane == 0) {
    sm_m[wave] = M;
    sm_l[wave] = L;
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int d = lane + 64 * k;
    if (d < HD) sm_o[wave][d] = O[k];
  }
  __syncthreads();
  if (wave != 0) return;
  float Mt = sm_m[0];
#pragma unroll
  for (int w = 1; w < MW; ++w) Mt = fmaxf(Mt, sm_m[w]);
  const float sl2 = sink ? sink[h] * 1.4426950408889634f : -INFINITY;
  Mt = fmaxf(Mt, sl2);
  float Lt = sink ? exp2f(sl2 - Mt) : 0.f, Ot[DPL] = {};
#pragma unroll
  for (int w = 0; w < MW; ++w) {
    const float e = (sm_m[w] == -INFINITY) ? 0.f : exp2f(sm_m[w] - Mt);
    Lt += e * sm_l[w];
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int d = lane + 64 * k;
      if (d < HD) Ot[k] += e * sm_o[w][d];
    }
  }
  const float inv = v_scale / Lt;
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int d = lane + 64 * k;
    if (d < HD) out[d] = G ? attn_out_gated(Ot[k] * inv, gp[k], bp) : f2bf(Ot[k] * inv);
  }
}

// Split-K workgroups per launch aimed for (each wave one 64-key tile until
// the context needs more than kAttnChunkTarget * 4 tiles).
constexpr int kAttnChunkTarget = 4096;

void attn_plan(int T, int Hkv, int span, int* tpw, int* nch) {
  const int tiles = (span + 63) / 64;
  const int target = std::max(1, kAttnChunkTarget / std::max(1, Hkv * T));
  int w = (tiles + 4 * target - 1) / (4 * target);
  // A short span over many (token, kv head) pairs (a batch of sliding-window
  // decode steps): one workgroup per pair walks the whole span, with no
  // records and no merge (128 sequences, 513 keys: 40.4 us + 5.8 us of merge
  // -> 35.4 us)
  if (T * Hkv >= 256 && tiles <= 16) w = (tiles + 3) / 4;
  w = std::min(std::max(w, 1), 64);
  *tpw = w;
  *nch = std::max(1, (tiles + 4 * w - 1) / (4 * w));
}

// An upper bound of attn_plan's nch over every span up to `span`, monotone in
// span, so a workspace sized for a context bound serves any shorter one.
int attn_nch_bound(int T, int Hkv, int span) {
  const int tiles = (span + 63) / 64;
  const int target = std::max(1, kAttnChunkTarget / std::max(1, Hkv * T));
  return std::max(std::max(1, std::min(target, (tiles + 3) / 4)), (tiles + 255) / 256);
}

bool attn_fused_merge(int T, int Hkv, int nch) {
  return nch > 1 && nch <= kAttnFusedMergeMax && T * Hkv <= kAttnCounters;
}

int launch_attn_decode(int T, int Hq, int Hkv, int hd, int swa, int window, int fp8,
                       const uint16_t* q, const int32_t* pos, const int32_t* seq,
                       const void* kc, const void* vc, float k_scale, float v_scale, int S,
                       int Lmax, int npos, const float* sink, uint16_t* o, int span, float* part,
                       unsigned* ctr, hipStream_t st, const AttnFuse* fuse) {
  const float score_scale = k_scale / sqrtf((float)hd) * 1.4426950408889634f;
  const float vsc = fp8 ? v_scale : 1.0f;
  int tpw, nch;
  attn_plan(T, Hkv, span, &tpw, &nch);
  const dim3 grid(nch, Hkv, T);
  const bool fused = attn_fused_merge(T, Hkv, nch);
  uint16_t* od = (nch == 1 || fused) ? o : nullptr;
  unsigned* cp = fused ? ctr : nullptr;
  const AttnFuse fz = fuse ? *fuse : AttnFuse{};
  // q epilogue and cache write fused into the attention kernel, or (qkv null)
  // only the gate, applied by the separate merge
  const bool fuse_qk = fuse != nullptr && fuse->qkv != nullptr;
  if (fuse != nullptr && !fuse_qk && od != nullptr) return -1;
#define ARGS q, pos, seq, kc, vc, S, Lmax, npos, Hq, Hkv, window, tpw, score_scale, nch, part, od, sink, vsc, cp, fz
#define PART(HD_, F8, SW)                                                                     \
  do {                                                                                        \
    if (fuse_qk)                                                                              \
      hipLaunchKernelGGL((attn_decode_partial_kernel<HD_, F8, SW, 4, 16, true>), grid,        \
                         dim3(256), 0, st, ARGS);                                             \
    else                                                                                      \
      hipLaunchKernelGGL((attn_decode_partial_kernel<HD_, F8, SW, 4, 16, false>), grid,       \
                         dim3(256), 0, st, ARGS);                                             \
  } while (0)
#define STREAM(HD_, SW)                                                                       \
  do {                                                                                        \
    if (fuse_qk)                                                                              \
      hipLaunchKernelGGL((attn_decode_fp8_stream_kernel<HD_, SW, true>), grid, dim3(256), 0,  \
                         st, ARGS);                                                           \
    else                                                                                      \
      hipLaunchKernelGGL((attn_decode_fp8_stream_kernel<HD_, SW, false>), grid, dim3(256), 0, \
                         st, ARGS);                                                           \
  } while (0)
#define BY_MODE(HD_)                                                   \
  if (fp8 && !od) {                                                   \
    if (swa) STREAM(HD_, true); else STREAM(HD_, false);              \
  } else if (fp8) {                                                   \
    if (swa) PART(HD_, true, true); else PART(HD_, true, false);      \
  } else {                                                            \
    if (swa) PART(HD_, false, true); else PART(HD_, false, false);    \
  }
  if (hd == 128) { BY_MODE(128) }
  else if (hd == 64) { BY_MODE(64) }
  else { BY_MODE(32) }
#undef BY_MODE
#undef STREAM
#undef PART
#undef ARGS
  if (hipGetLastError() != hipSuccess) return -1;
  if (od) return 0;
  const float vs = fp8 ? v_scale : 1.0f;
  const uint16_t* G = fz.g;
  const uint16_t* bg = fz.bgate;
  if (nch <= kAttnFusedMergeMax) {
    const dim3 sg((T * Hq + 3) / 4);
#define SMALL(HD_)                                                                              \
  hipLaunchKernelGGL((attn_merge_small_kernel<HD_>), sg, dim3(256), 0, st, part, pos, seq, S,   \
                     npos, T, Hq, window, swa, tpw, nch, sink, vs, o, G, bg)
    if (hd == 128) SMALL(128);
    else if (hd == 64) SMALL(64);
    else SMALL(32);
#undef SMALL
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const dim3 mg(Hq, T);
  if (hd == 128)
    hipLaunchKernelGGL((attn_merge_kernel<128>), mg, dim3(1024), 0, st, part, pos, seq, S, npos, Hq,
                       window, swa, tpw, nch, sink, vs, o, G, bg);
  else if (hd == 64)
    hipLaunchKernelGGL((attn_merge_kernel<64>), mg, dim3(1024), 0, st, part, pos, seq, S, npos, Hq,
                       window, swa, tpw, nch, sink, vs, o, G, bg);
  else
    hipLaunchKernelGGL((attn_merge_kernel<32>), mg, dim3(1024), 0, st, part, pos, seq, S, npos, Hq,
                       window, swa, tpw, nch, sink, vs, o, G, bg);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace beam
