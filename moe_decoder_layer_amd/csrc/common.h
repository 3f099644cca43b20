// Device helpers shared by the libbeamlayer kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;

// ---- bf16 <-> fp32 -------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float round_bf(float f) { return bf2f(f2bf(f)); }
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// ---- fp8 e4m3fn (OCP) ------------------------------------------------------
// Encode with round-to-nearest-even and saturation at +-448 (NaN -> 0x7f).
__device__ __forceinline__ uint8_t f2e4m3(float x) {
  uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  if (!(a == a)) return 0x7f;
  a = fminf(a, 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                      // below 2^-6: subnormal grid of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);  // 8 rounds up into the first normal
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7ffffu + ((b >> 20) & 1u);       // keep 3 mantissa bits, ties to even
    code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  }
  return (uint8_t)(code | sign);
}
// Four fp8 codes of a 32-bit word -> four bf16 (exact; gfx950 packed
// conversion, unit scale, low byte pair then high byte pair).
__device__ __forceinline__ bf16x4 e4m3x4_to_bf16x4(uint32_t w) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
  return bf16x4{a[0], a[1], b[0], b[1]};
}
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint2 w) {
  bf16x4 a = e4m3x4_to_bf16x4(w.x), b = e4m3x4_to_bf16x4(w.y);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ---- loads -----------------------------------------------------------------
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Streaming (non-temporal) 16-byte load for weights read once per step.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ f32x4 ld16f_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 bf16 . 8 bf16 accumulated in fp32.
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
  acc = __builtin_fmaf(bf_lo(a.x), bf_lo(b.x), acc);
  acc = __builtin_fmaf(bf_hi(a.x), bf_hi(b.x), acc);
  acc = __builtin_fmaf(bf_lo(a.y), bf_lo(b.y), acc);
  acc = __builtin_fmaf(bf_hi(a.y), bf_hi(b.y), acc);
  acc = __builtin_fmaf(bf_lo(a.z), bf_lo(b.z), acc);
  acc = __builtin_fmaf(bf_hi(a.z), bf_hi(b.z), acc);
  acc = __builtin_fmaf(bf_lo(a.w), bf_lo(b.w), acc);
  acc = __builtin_fmaf(bf_hi(a.w), bf_hi(b.w), acc);
  return acc;
}

// The same sum with gfx950's packed bf16 dot product (two products and the
// accumulator per instruction, fp32 result): no unpacking of either operand.
// bf16 x bf16 products are exact in fp32; only the summation order differs
// from dot8_bf16.
__device__ __forceinline__ float dot8_bf16_d2(uint4 a, uint4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x),
                                        __builtin_bit_cast(bf16x2, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y),
                                        __builtin_bit_cast(bf16x2, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z),
                                        __builtin_bit_cast(bf16x2, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w),
                                        __builtin_bit_cast(bf16x2, b.w), acc, false);
  return acc;
}

// ---- wave reductions (wave64) ------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// 16 bytes per lane from global memory straight into LDS (gfx950): a wave
// writes 64 x 16 B contiguously from the wave-uniform LDS address `lds`. The
// builtin exists only in the device pass; the host pass compiles an empty body
// so that it still emits the kernels' launch stubs.
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
#endif
}
// The same with 4 bytes per lane (64 x 4 B written contiguously).
__device__ __forceinline__ void load_lds4(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
#endif
}

// ---- last-arriver election ---------------------------------------------------
// Workgroups that each publish partial results and then need one of them to
// combine everything. Published values are written with st_dev: a relaxed
// device-scope store, which goes through to the device's coherence point
// instead of staying in this XCD's L2, so no L2 write-back is needed. Each wave
// waits for its own stores to complete, the workgroup meets at a barrier, and
// one relaxed device-scope atomic per workgroup counts arrivals. Returns true
// (uniformly) in the workgroup that arrives last; it resets the counter for
// the next launch and, after an acquire fence, reads what the others
// published. No workgroup ever waits on another, so nothing can hang.
// *ctr must be zero when the launch starts.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool last_arrival(unsigned* ctr, unsigned nblocks, int* sflag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (old == nblocks - 1u);
    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sflag = last;
  }
  __syncthreads();
  const bool last = *sflag != 0;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

// ---- math ------------------------------------------------------------------
// exp and reciprocal on the transcendental unit (about 1 ulp each in fp32),
// instead of an IEEE division sequence: these run once per activation element
// in the gate and SwiGLU epilogues, where a division would cost ~10 VALU ops.
__device__ __forceinline__ float sigmoidf_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
__device__ __forceinline__ float siluf(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// ---- device-side argument checks ---------------------------------------------
// Each translation unit that checks data-dependent indices owns one flag.
#define BEAM_ERR_FLAG_DECL(tu) static __device__ int tu##_err_flag;
#define BEAM_RAISE(tu, bit) atomicOr(&tu##_err_flag, (bit))
#define BEAM_ERR_FLAG_READER(tu)                                                 \
  int tu##_read_clear_err() {                                                    \
    int v = 0, z = 0;                                                            \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(tu##_err_flag), sizeof(int)) != hipSuccess) \
      return -1;                                                                 \
    if (hipMemcpyToSymbol(HIP_SYMBOL(tu##_err_flag), &z, sizeof(int)) != hipSuccess) \
      return -1;                                                                 \
    return v;                                                                    \
  }

// ERR_SPAN: a token's position lies beyond the max_pos its call was sized for.
// ERR_RANGE: a value outside the range of an intermediate format (the prefill
// attention's fp16 P.V operand) was clamped.
enum : int { ERR_POS = 1, ERR_SEQ = 2, ERR_EXPERT = 4, ERR_SPAN = 8, ERR_RANGE = 16 };

}  // namespace beam
