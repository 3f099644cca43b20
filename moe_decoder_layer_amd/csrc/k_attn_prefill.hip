// Many-token GQA attention over the KV cache (chunked prefill): causal inside
// the chunk, sliding window on SWA layers, full context on NoPE layers
// ("Reflection Beam 1.0 on vLLM", Attention section). The chunk's own keys
// were written to the cache first, so every token reads keys
// [lo_t, p_t] of its sequence from the cache alone.
//
// Workgroup = (block of 32 consecutive tokens, kv head j); wave w is query
// head j * grp + w, so the group's waves read the same K/V lines (shared
// through the CU's L1). Per 32-key block and wave, on 32x32x16 bf16 MFMA:
//   S^T[key][token] = K[key][:] . Q[token][:]
//   O^T[dim][token] += V^T[dim][key] . P^T[key][token]   (P as hi + lo bf16)
// In the S^T layout lane l owns token l % 32, so the online softmax state is
// lane-local up to one xor-32 shuffle, and a lane's probabilities are the B
// operand it needs for P.V. Keys are visited in the union of the 32 tokens'
// ranges; per-token masks cut each token's own range, and value rows outside
// the union are zeroed before they can meet a zero probability.
// Tokens of several sequences in one block are handled in one pass per
// sequence.
#include "common.h"
#include "internal.h"

namespace beam {

template <int HD, bool FP8, bool SWA>
__global__ __launch_bounds__(512) void attn_prefill_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ seq, const void* __restrict__ kc, const void* __restrict__ vc,
    int S, int Lmax, int Hq, int Hkv, int window, float score_scale, int T,
    const float* __restrict__ sink, float v_scale, uint16_t* __restrict__ o) {
  constexpr int KS = HD / 16;  // k-steps of the score product (16 dims each)
  constexpr int DB = HD / 32;  // 32-dim blocks of the output
  constexpr int LD = HD / 2;   // dims per lane half in the score product
  const int j = blockIdx.y;
  const int grp = Hq / Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = j * grp + wave;
  const int tc = lane & 31, g = lane >> 5;
  const int t = blockIdx.x * 32 + tc;
  const bool tok = t < T;
  int p = tok ? pos[t] : -1;
  int s = tok ? seq[t] : -1;
  if (p < 0 || p >= Lmax || s < 0 || s >= S) {  // invalid tokens attend nothing
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
    // next sequence present in the block (ascending), and its key range
    int s_cur = (s > s_prev) ? s : 0x7fffffff;
    for (int o2 = 32; o2 > 0; o2 >>= 1) s_cur = min(s_cur, __shfl_xor(s_cur, o2, 64));
    if (s_cur == 0x7fffffff) break;
    s_prev = s_cur;
    const bool mine = (s == s_cur);
    int kmin = mine ? lo : 0x7fffffff, kmax = mine ? p : -1;
    for (int o2 = 32; o2 > 0; o2 >>= 1) {
      kmin = min(kmin, __shfl_xor(kmin, o2, 64));
      kmax = max(kmax, __shfl_xor(kmax, o2, 64));
    }
    const size_t krow0 = ((size_t)s_cur * Hkv + j) * (size_t)Lmax;
    const size_t vrow0 = ((size_t)s_cur * Hkv + j) * (size_t)HD;
    for (int kb = kmin & ~31; kb <= kmax; kb += 32) {
      f32x16 sacc = f32x16{};
      const size_t kr = (krow0 + kb + tc) * HD + g * LD;
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        bf16x8 kf;
        if constexpr (FP8) {
          kf = e4m3x8_to_bf16x8(*reinterpret_cast<const uint2*>((const uint8_t*)kc + kr + i * 8));
        } else {
          kf = as_bf16x8(ld16((const uint16_t*)kc + kr + i * 8));
        }
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[i], sacc, 0, 0, 0);
      }
      // sacc[4 i + jj] = S[key kb + 8 i + 4 g + jj][token tc]
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int key = kb + 8 * i + 4 * g + jj;
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
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      const bool edge = (kb < kmin) || (kb + 31 > kmax);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 ph, pl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float pv = sacc[4 * (2 * st + (i >> 2)) + (i & 3)];
          ph[i] = (__bf16)pv;
          pl[i] = (__bf16)(pv - (float)ph[i]);
        }
        const int key0 = kb + 16 * st + 4 * g, key1 = key0 + 8;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const size_t vr = (vrow0 + db * 32 + tc) * (size_t)Lmax;
          bf16x8 vf;
          if constexpr (FP8) {
            const uint8_t* vb = (const uint8_t*)vc + vr;
            const bf16x4 a = e4m3x4_to_bf16x4(*reinterpret_cast<const uint32_t*>(vb + key0));
            const bf16x4 b = e4m3x4_to_bf16x4(*reinterpret_cast<const uint32_t*>(vb + key1));
            vf = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
          } else {
            const uint16_t* vb = (const uint16_t*)vc + vr;
            const uint2 a = *reinterpret_cast<const uint2*>(vb + key0);
            const uint2 b = *reinterpret_cast<const uint2*>(vb + key1);
            vf = __builtin_bit_cast(bf16x8, uint4{a.x, a.y, b.x, b.y});
          }
          if (edge) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int key = (i < 4 ? key0 + i : key1 + i - 4);
              if (key < kmin || key > kmax) vf[i] = (__bf16)0.0f;
            }
          }
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, ph, oacc[db], 0, 0, 0);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl, oacc[db], 0, 0, 0);
        }
      }
    }
  }
  if (!tok) return;
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

int launch_attn_prefill(int T, int Hq, int Hkv, int hd, int swa, int window, int fp8,
                        const uint16_t* q, const int32_t* pos, const int32_t* seq,
                        const void* kc, const void* vc, float k_scale, float v_scale, int S,
                        int Lmax, const float* sink, uint16_t* o, hipStream_t st) {
  const float score_scale = k_scale / sqrtf((float)hd) * 1.4426950408889634f;
  const int grp = Hq / Hkv;
  const dim3 grid((T + 31) / 32, Hkv), block(64 * grp);
  const float vs = fp8 ? v_scale : 1.0f;
#define PF(HD_, F8, SW)                                                                      \
  hipLaunchKernelGGL((attn_prefill_kernel<HD_, F8, SW>), grid, block, 0, st, q, pos, seq, kc, \
                     vc, S, Lmax, Hq, Hkv, window, score_scale, T, sink, vs, o)
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
