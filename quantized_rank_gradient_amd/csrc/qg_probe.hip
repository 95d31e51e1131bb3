// Calibration of the compute roofline: the bf16 MFMA rate the chip sustains on given operand
// data. The published dense bf16 peak assumes the full clock; under sustained MFMA load the
// clock and hence the rate depend on the switching activity of the operands, so the rate is
// measured on random operands (like the step's gradients and projections) and on constant
// ones. Every wave reads 4 A and 4 B fragments once from the caller's buffer and then runs
// `iters` rounds of 16 independent v_mfma_f32_32x32x16_bf16 into 16 accumulator blocks;
// nothing but the products touches memory or the register file in the timed loop.
#include "qg_kernels.hpp"
#include "qg_device.hpp"

namespace qg {

__global__ __launch_bounds__(kThreads, 1) void qg_mfma_probe(const bf16x8* src, uint32_t nfrag,
                                                            float* out, int iters) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    a[x] = src[(t * 8 + x) % nfrag];
    b[x] = src[(t * 8 + 4 + x) % nfrag];
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y)
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], b[y], acc[x][y], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[x][y][v];
  out[t] = s;
}

hipError_t launch_mfma_probe(const uint16_t* operands, int64_t n_elems, float* out, int grid,
                             int iters, hipStream_t s) {
  hipLaunchKernelGGL(qg_mfma_probe, dim3(grid), dim3(kThreads), 0, s,
                     reinterpret_cast<const bf16x8*>(operands), (uint32_t)(n_elems / 8), out,
                     iters);
  return hipGetLastError();
}

}  // namespace qg
