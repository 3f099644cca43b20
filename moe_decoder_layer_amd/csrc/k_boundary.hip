// Sublayer boundary: post-norm -> depth-scaled residual add -> next pre-norm,
// one kernel per boundary ("Reflection Beam 1.0 on vLLM", MoE and residual
// stream section for the maths; optimisation change 1 for the fusion).
//
// One workgroup per token row. The row is held in registers between the two
// RMS reductions: 256 threads x up to 4 chunks of 8 bf16 covers D <= 8192.
// All statistics are fp32; every stored tensor is bf16.
#include "boundary_row.h"
#include "common.h"
#include "internal.h"

namespace beam {

constexpr int BT = 256;
constexpr int CPT = 4;  // 16-byte chunks per thread (D <= BT * CPT * 8)

__global__ __launch_bounds__(BT) void boundary_kernel(
    int D, const uint16_t* __restrict__ y, const uint16_t* __restrict__ w_post,
    uint16_t* __restrict__ h, const uint16_t* __restrict__ w_pre,
    uint16_t* __restrict__ x_out, int mode, float c_h, float c_a, float eps) {
  __shared__ float red[BT / 64];
  const size_t row = (size_t)blockIdx.x * D;
  BoundaryRow<BT, CPT> b;
  b.load(D, y ? y + row : nullptr, w_post, h + row, w_pre, mode);
  uint4 hn[CPT], xo[CPT];
  b.compute(D, mode, c_h, c_a, eps, red, hn, xo);
  const int nc = D >> 3;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * BT;
    if (c < nc) {
      if (mode != 0) *reinterpret_cast<uint4*>(h + row + c * 8) = hn[i];
      *reinterpret_cast<uint4*>(x_out + row + c * 8) = xo[i];
    }
  }
}

int launch_boundary(int T, int D, const uint16_t* y, const uint16_t* w_post, uint16_t* h,
                    const uint16_t* w_pre, uint16_t* x_out, int n, float eps,
                    hipStream_t st) {
  const int mode = (y == nullptr) ? 0 : (w_post != nullptr ? 1 : 2);
  float c_h, c_a;
  boundary_coefs(mode == 0 ? 0 : n, &c_h, &c_a);
  hipLaunchKernelGGL(boundary_kernel, dim3(T), dim3(BT), 0, st, D, y, w_post, h, w_pre,
                     x_out, mode, c_h, c_a, eps);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace beam
